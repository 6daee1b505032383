"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments before anything is enqueued.  No kernel is launched."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

SPEC_OK, SPEC_EINVAL, SPEC_EDTYPE, SPEC_EWORKSPACE, SPEC_EHIP, SPEC_ESCRATCH = range(6)


@pytest.fixture(scope="module")
def lib():
    return sv.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) >= {"spec_verify_greedy", "spec_verify_exact", "spec_verify_relaxed",
                          "spec_verify_tree", "spec_verify_workspace_bytes", "spec_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(6):
        assert lib.spec_status_string(code)
    assert b"scratch" in lib.spec_status_string(5)
    assert b"unknown" in lib.spec_status_string(99)


def test_noalloc_argument_errors(lib):
    """The allocation-free exact call rejects bad arguments, and calls whose
    workspace would exceed the 4 MiB static scratch array, before anything
    is enqueued (and before the array's address is looked up)."""
    f = lib.spec_verify_exact_noalloc
    p = P4K
    assert f(p, p, 7, p, p, 2, 3, 1000, p, p, None, None, p, None) == SPEC_EDTYPE
    assert f(p, None, 1, p, p, 2, 3, 1000, p, p, None, None, p, None) == SPEC_EINVAL
    assert f(p, p, 1, p, p, 2, 64, 1000, p, p, None, None, p, None) == SPEC_EINVAL
    assert f(p, p, 1, p, p, 2, 3, 1000, None, p, None, None, p, None) == SPEC_EINVAL
    limit = 4 << 20
    q = lib.spec_verify_workspace_bytes
    assert q(128, 17, 262144) <= limit           # the documented example fits
    assert q(1024, 11, 262144) > limit
    assert f(p, p, 0, p, p, 1024, 5, 262144, p, p, None, None, p, None) == SPEC_ESCRATCH
    assert f(p, p, 1, p, p, 4096, 5, 128256, p, p, None, None, p, None) == SPEC_ESCRATCH


def test_workspace_query(lib):
    q = lib.spec_verify_workspace_bytes
    assert q(0, 6, 100) == 0 and q(1, 0, 100) == 0 and q(1, 6, 0) == 0 and q(1, 128, 10) == 0
    assert q(65537, 6, 100) == 0
    a, b, c = q(8, 6, 128256), q(32, 11, 128256), q(32, 11, 151936)
    assert 0 < a < b < c
    assert a % 256 == 0
    assert a >= 8 * 6 * 32 * 16  # one 16-byte record per (row, tile) at fp32 tiles


ws_buf = (ctypes.c_uint8 * 64)()  # host memory: only its address is inspected
P4K = ctypes.c_void_p(4096)
PWS = ctypes.c_void_p(1 << 20)


def _greedy(lib, **over):
    args = dict(T=ctypes.c_void_p(4096), dt=1, x=ctypes.c_void_p(4096), B=2, K=3, V=100,
                tok=ctypes.c_void_p(4096), ln=ctypes.c_void_p(4096), tlp=None, blp=None,
                st=ctypes.c_void_p(4096), ws=ctypes.c_void_p(1 << 20), wsb=0, stream=None)
    args.update(over)
    return lib.spec_verify_greedy(*args.values())


def test_greedy_argument_errors(lib):
    assert _greedy(lib, dt=2) == SPEC_EDTYPE
    assert _greedy(lib, B=0) == SPEC_EINVAL
    assert _greedy(lib, K=0) == SPEC_EINVAL
    assert _greedy(lib, K=64) == SPEC_EINVAL
    assert _greedy(lib, V=0) == SPEC_EINVAL
    assert _greedy(lib, T=None) == SPEC_EINVAL
    assert _greedy(lib, x=None) == SPEC_EINVAL
    assert _greedy(lib, st=None) == SPEC_EINVAL
    assert _greedy(lib, ws=None) == SPEC_EWORKSPACE
    assert _greedy(lib, ws=ctypes.c_void_p((1 << 20) + 8)) == SPEC_EWORKSPACE  # misaligned
    need = lib.spec_verify_workspace_bytes(2, 4, 100)
    assert _greedy(lib, wsb=need - 256) == SPEC_EWORKSPACE                      # too small


def test_streaming_grid_limit(lib):
    # one 256-thread workgroup per 16 KiB tile, at most 2^32 threads a launch:
    # B * (K + 1) * tiles < 2^24.  bf16 V = 262144 has 32 tiles a row, fp32 64.
    big = dict(B=65536, V=262144)
    assert _greedy(lib, K=7, **big) == SPEC_EINVAL                  # 2^24 bf16 tiles
    assert _greedy(lib, K=6, **big) == SPEC_EWORKSPACE              # sizes pass, no workspace
    assert _greedy(lib, dt=0, K=3, **big) == SPEC_EINVAL            # 2^24 fp32 tiles
    assert _greedy(lib, dt=0, K=2, **big) == SPEC_EWORKSPACE


def test_exact_relaxed_tree_argument_errors(lib):
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)
    need = lib.spec_verify_workspace_bytes(2, 7, 100)
    # exact: missing draft logits, missing uniforms
    assert lib.spec_verify_exact(p, None, 1, p, p, 2, 3, 100, p, p, None, None, p, ws, need,
                                 None) == SPEC_EINVAL
    assert lib.spec_verify_exact(p, p, 1, p, None, 2, 3, 100, p, p, None, None, p, ws, need,
                                 None) == SPEC_EINVAL
    assert lib.spec_verify_exact(p, p, 9, p, p, 2, 3, 100, p, p, None, None, p, ws, need,
                                 None) == SPEC_EDTYPE
    # relaxed: NaN tau, negative top_k
    assert lib.spec_verify_relaxed(p, 1, p, p, 2, 3, 100, ctypes.c_float(float("nan")), 4, p, p,
                                   None, None, p, ws, need, None) == SPEC_EINVAL
    assert lib.spec_verify_relaxed(p, 1, p, p, 2, 3, 100, ctypes.c_float(0.1), -1, p, p, None,
                                   None, p, ws, need, None) == SPEC_EINVAL
    # tree: N out of range, missing parents
    assert lib.spec_verify_tree(p, 1, p, p, None, 2, 65, 100, p, p, p, None, None, p, ws, need,
                                None) == SPEC_EINVAL
    assert lib.spec_verify_tree(p, 1, p, None, None, 2, 8, 100, p, p, p, None, None, p, ws, need,
                                None) == SPEC_EINVAL
    assert lib.spec_verify_tree(p, 1, p, p, None, 2, 8, 100, p, p, p, None, None, p, ws, 16,
                                None) == SPEC_EWORKSPACE


def test_binding_rejects_host_tensors():
    T = torch.zeros((2, 4, 50), dtype=torch.bfloat16)
    x = torch.zeros((2, 3), dtype=torch.int32)
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_greedy(T, x)
    with pytest.raises(sv.SpecVerifyError):
        sv.spec_verify_exact(T, T[:, :3], x, torch.zeros((2, 4)))


def test_header_has_no_torch_or_hip_types():
    src = open(HEADER).read()
    assert "torch" not in src.lower().replace("torch tensors", "")
    assert "#include <hip" not in src


def test_power_and_sampler_argument_errors(lib):
    p = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(1 << 20)
    need = lib.spec_verify_workspace_bytes(2, 7, 100)
    F = ctypes.c_float
    # power: negative, NaN and infinite alpha; missing draft logits
    for alpha in (-0.5, float("nan"), float("inf")):
        assert lib.spec_verify_power(p, p, 1, p, p, 2, 3, 100, F(alpha), p, p, None, None, p, ws,
                                     need, None) == SPEC_EINVAL
    assert lib.spec_verify_power(p, None, 1, p, p, 2, 3, 100, F(1.0), p, p, None, None, p, ws, need,
                                 None) == SPEC_EINVAL
    assert lib.spec_verify_power(p, p, 1, p, p, 2, 3, 100, F(1.0), p, p, None, None, p, ws, 64,
                                 None) == SPEC_EWORKSPACE
    # sampler: bad rows, missing uniforms, small workspace
    wsz = lib.spec_sample_workspace_bytes(10, 100)
    assert wsz > 0 and lib.spec_sample_workspace_bytes(0, 100) == 0
    assert lib.spec_sample_drafts(p, 1, p, 0, 100, p, None, p, ws, wsz, None) == SPEC_EINVAL
    assert lib.spec_sample_drafts(p, 1, None, 10, 100, p, None, p, ws, wsz, None) == SPEC_EINVAL
    assert lib.spec_sample_drafts(p, 1, p, 10, 100, p, None, p, ws, wsz - 256, None) == SPEC_EWORKSPACE



def test_shard_size_queries(lib):
    rb, sb, wb = lib.spec_shard_record_bytes, lib.spec_shard_sums_bytes, lib.spec_shard_workspace_bytes
    # 32 requests x 11 rows x 2 bf16 tiles of 16032 columns, then the drafted-token logits
    assert rb(1, 32, 11, 128256, 8) == 14080
    assert rb(1, 32, 11, 128256, 7) == 0        # 128256 is not a multiple of 7
    assert rb(1, 32, 11, 128256, 0) == 0
    assert rb(2, 32, 11, 128256, 8) == 0        # bad dtype
    assert rb(1, 0, 11, 128256, 8) == 0 and rb(1, 32, 128, 128256, 8) == 0
    assert rb(0, 2, 13, 262144, 64) > 0         # fp32, one tile per shard row
    assert rb(0, 2, 13, 262144, 128) == 0       # 128 shard slots exceed one wave
    assert rb(1, 2, 13, 262144, 16) > 0         # 16 x 4 chunks: exactly one wave
    assert rb(1, 2, 13, 33 * 4100, 33) == 0     # 33 x 2 chunks exceed one wave
    assert sb(32, 128256, 8) == 32 * 4 * 48 and sb(32, 128256, 7) == 0  # 48-byte chunk records
    assert wb(32) == 2048 and wb(0) == 0
    for v in (rb(1, 32, 11, 128256, 8), sb(32, 128256, 8), wb(32)):
        assert v % 256 == 0




def test_shard_argument_errors(lib):
    rec = lib.spec_shard_record_bytes(1, 2, 7, 1000, 4)

    def stats(**over):
        a = dict(T=P4K, D=P4K, dt=1, x=P4K, B=2, K=3, V=1000, G=4, s=0, rec=PWS, rb=rec, st=None)
        a.update(over)
        return lib.spec_shard_stats_exact(*a.values())

    assert stats(dt=5) == SPEC_EDTYPE
    assert stats(G=3) == SPEC_EINVAL           # 1000 % 3 != 0
    assert stats(s=4) == SPEC_EINVAL and stats(s=-1) == SPEC_EINVAL
    assert stats(K=0) == SPEC_EINVAL
    assert stats(D=None) == SPEC_EINVAL and stats(x=None) == SPEC_EINVAL
    assert stats(rec=None) == SPEC_EWORKSPACE
    assert stats(rec=ctypes.c_void_p((1 << 20) + 16)) == SPEC_EWORKSPACE
    assert stats(rb=rec - 256) == SPEC_EWORKSPACE
    g = lib.spec_shard_stats_greedy
    assert g(P4K, 1, 2, 3, 1000, 4, 4, 1, PWS, 1 << 20, None) == SPEC_EINVAL   # shard = G
    t = lib.spec_shard_stats_tree
    assert t(P4K, 1, None, 2, 65, 1000, 4, 0, 1, PWS, 1 << 20, None) == SPEC_EINVAL  # N > 64
    cg = lib.spec_shard_combine_greedy
    grec = 4 * lib.spec_shard_record_bytes(1, 2, 4, 1000, 4)   # G gathered greedy slots
    assert cg(ctypes.c_void_p((1 << 20) + 64), grec, 1, P4K, 2, 3, 1000, 4, P4K, P4K, None, None,
              P4K, None) == SPEC_EWORKSPACE
    assert cg(PWS, grec, 1, None, 2, 3, 1000, 4, P4K, P4K, None, None, P4K, None) == SPEC_EINVAL
    ct = lib.spec_shard_combine_tree
    assert ct(PWS, 1 << 30, 1, P4K, None, None, 2, 8, 1000, 4, P4K, P4K, P4K, None, None, P4K,
              None) == SPEC_EINVAL
    sw = lib.spec_shard_sweep_exact
    sums, ws = lib.spec_shard_sums_bytes(2, 1000, 4), lib.spec_shard_workspace_bytes(2)
    base = [P4K, P4K, 1, PWS, 4 * rec, P4K, P4K, 2, 3, 1000, 4, 1, P4K, P4K, None, None, P4K, PWS,
            sums, PWS, ws, None]
    bad_sums = list(base)
    bad_sums[18] = sums - 256
    assert sw(*bad_sums) == SPEC_EWORKSPACE
    bad_ws = list(base)
    bad_ws[20] = 0
    assert sw(*bad_ws) == SPEC_EWORKSPACE
    bad_u = list(base)
    bad_u[6] = None
    assert sw(*bad_u) == SPEC_EINVAL
    sa = lib.spec_shard_sample_exact
    assert sa(P4K, P4K, 1, ctypes.c_void_p((1 << 20) + 32), 4 * sums, P4K, 2, 3, 1000, 4, 1, P4K,
              None, None, None, PWS, ws, None) == SPEC_EWORKSPACE
    assert sa(P4K, P4K, 1, PWS, 4 * sums, P4K, 2, 3, 1000, 4, 9, P4K, None, None, None, PWS, ws,
              None) == SPEC_EINVAL


def test_shard_gathered_inputs_are_size_checked(lib):
    """Every gathered input (G record, sums or values slots) comes with its
    size; one byte short of G slots is rejected before anything is enqueued,
    and exactly G slots passes the check (the next error is the test's
    missing stream-side inputs, never a launch)."""
    G, B, K, V = 4, 2, 3, 1000
    ws = lib.spec_shard_workspace_bytes(B)
    sums = lib.spec_shard_sums_bytes(B, V, G)
    rec_pq = lib.spec_shard_record_bytes(1, B, 2 * K + 1, V, G)
    rec_g = lib.spec_shard_record_bytes(1, B, K + 1, V, G)
    rec_t = lib.spec_shard_record_bytes(1, B, 8, V, G)
    vals = lib.spec_shard_values_bytes(B, K)
    f = ctypes.c_float
    # argument lists with every pointer valid and the gathered input's size n,
    # and the same with a required output (or the logits) missing
    calls = {
        "combine_greedy": (lib.spec_shard_combine_greedy, G * rec_g,
                           lambda n, o: [PWS, n, 1, P4K, B, K, V, G, P4K, P4K, None, None, o, None]),
        "combine_tree": (lib.spec_shard_combine_tree, G * rec_t,
                         lambda n, o: [PWS, n, 1, P4K, P4K, None, B, 8, V, G, P4K, P4K, P4K, None,
                                       None, o, None]),
        "sweep_exact": (lib.spec_shard_sweep_exact, G * rec_pq,
                        lambda n, o: [P4K, P4K, 1, PWS, n, P4K, P4K, B, K, V, G, 1, P4K, P4K, None,
                                      None, o, PWS, sums, PWS, ws, None]),
        "sweep_power": (lib.spec_shard_sweep_power, G * rec_pq,
                        lambda n, o: [P4K, P4K, 1, PWS, n, P4K, P4K, B, K, V, G, 1, f(0.5), P4K, P4K,
                                      None, None, o, PWS, sums, PWS, ws, None]),
        "sweep_relaxed": (lib.spec_shard_sweep_relaxed, G * rec_g,
                          lambda n, o: [P4K, 1, PWS, n, P4K, P4K, B, K, V, G, 0, f(0.1), 4, P4K, P4K,
                                        None, None, o, PWS, sums, PWS, ws, None]),
        "sample_exact": (lib.spec_shard_sample_exact, G * sums,
                         lambda n, o: [P4K, P4K, 1, PWS, n, P4K, B, K, V, G, 1, o, None, None, None,
                                       PWS, ws, None]),
        "sample_power": (lib.spec_shard_sample_power, G * sums,
                         lambda n, o: [P4K, P4K, 1, PWS, n, P4K, B, K, V, G, 1, o, None, None, None,
                                       PWS, ws, None]),
        "sample_relaxed": (lib.spec_shard_sample_relaxed, G * sums,
                           lambda n, o: [P4K, 1, PWS, n, P4K, B, K, V, G, 0, o, None, None, None,
                                         PWS, ws, None]),
        "stats_relaxed": (lib.spec_shard_stats_relaxed, G * vals,
                          lambda n, o: [o, 1, P4K, PWS, n, B, K, V, G, 0, PWS, 0, None]),
    }
    for name, (fn, need, args) in calls.items():
        assert need > 0, name
        # short by one byte, or empty: rejected whatever else is wrong
        assert fn(*args(need - 1, P4K)) == SPEC_EWORKSPACE, name
        assert fn(*args(0, None)) == SPEC_EWORKSPACE, name
        assert fn(*args(need - 1, None)) == SPEC_EWORKSPACE, name
        # G full slots pass the size check: the call stops at the missing
        # output instead
        assert fn(*args(need, None)) == SPEC_EINVAL, name


def test_read_ceiling_argument_errors(lib):
    w = lib.spec_read_ceiling_out_words
    assert w(0) == 0 and w(15) == 0 and w(24) == 0
    assert w(16) == 1 and w(16384) == 1 and w(16400) == 2
    r = lib.spec_read_ceiling
    assert r(None, 16384, P4K, None) == SPEC_EINVAL
    assert r(P4K, 16384, None, None) == SPEC_EINVAL
    assert r(P4K, 100, P4K, None) == SPEC_EINVAL                  # not a multiple of 16
    assert r(ctypes.c_void_p(4100), 16384, P4K, None) == SPEC_EINVAL  # misaligned


def test_shard_power_argument_errors(lib):
    sums, ws = lib.spec_shard_sums_bytes(2, 1000, 4), lib.spec_shard_workspace_bytes(2)
    base = [P4K, P4K, 1, PWS, 1 << 30, P4K, P4K, 2, 3, 1000, 4, 1, ctypes.c_float(0.5), P4K, P4K,
            None, None, P4K, PWS, sums, PWS, ws, None]
    for alpha in (-1.0, float("inf"), float("nan")):
        bad = list(base)
        bad[12] = ctypes.c_float(alpha)
        assert lib.spec_shard_sweep_power(*bad) == SPEC_EINVAL
    bad = list(base)
    bad[9] = 1001                     # not a multiple of G
    assert lib.spec_shard_sweep_power(*bad) == SPEC_EINVAL
    assert lib.spec_shard_sample_power(P4K, P4K, 1, PWS, 1 << 30, P4K, 2, 3, 1000, 4, 4, P4K, None,
                                       None, None, PWS, ws, None) == SPEC_EINVAL   # shard = G


def test_shard_relaxed_argument_errors(lib):
    assert lib.spec_shard_values_bytes(32, 5) == 768 and lib.spec_shard_values_bytes(0, 5) == 0
    assert lib.spec_shard_values_bytes(2, 64) == 0
    vb = lib.spec_shard_values_bytes(2, 3)
    v = lib.spec_shard_values_relaxed
    assert v(P4K, 1, P4K, 2, 3, 1000, 3, 0, PWS, vb, None) == SPEC_EINVAL      # 1000 % 3
    assert v(P4K, 1, None, 2, 3, 1000, 4, 0, PWS, vb, None) == SPEC_EINVAL
    assert v(P4K, 1, P4K, 2, 3, 1000, 4, 0, PWS, vb - 256, None) == SPEC_EWORKSPACE
    rb = lib.spec_shard_record_bytes(1, 2, 4, 1000, 4)
    st = lib.spec_shard_stats_relaxed
    assert st(P4K, 1, P4K, ctypes.c_void_p((1 << 20) + 8), 4 * vb, 2, 3, 1000, 4, 0, PWS, rb,
              None) == SPEC_EWORKSPACE
    assert st(P4K, 1, P4K, PWS, 4 * vb, 2, 3, 1000, 4, 4, PWS, rb, None) == SPEC_EINVAL   # shard = G
    assert st(P4K, 1, P4K, PWS, 4 * vb, 2, 3, 1000, 4, 0, PWS, rb - 256, None) == SPEC_EWORKSPACE
    sums, ws = lib.spec_shard_sums_bytes(2, 1000, 4), lib.spec_shard_workspace_bytes(2)
    sw = lib.spec_shard_sweep_relaxed
    base = [P4K, 1, PWS, 4 * rb, P4K, P4K, 2, 3, 1000, 4, 0, ctypes.c_float(0.1), 4, P4K, P4K, None,
            None, P4K, PWS, sums, PWS, ws, None]
    bad = list(base)
    bad[11] = ctypes.c_float(float("nan"))
    assert sw(*bad) == SPEC_EINVAL
    bad = list(base)
    bad[12] = -1
    assert sw(*bad) == SPEC_EINVAL
    sa = lib.spec_shard_sample_relaxed
    assert sa(P4K, 1, PWS, 4 * sums, None, 2, 3, 1000, 4, 0, P4K, None, None, None, PWS, ws,
              None) == SPEC_EINVAL
