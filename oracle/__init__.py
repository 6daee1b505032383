"""fp64 CPU oracle of the batched draft-verification sampler (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by the
smoke check in ``__graft_entry__`` and by the CPU-baseline leg of
``bench.py``; the product path (``draft_verification_row_amd``) never imports
it, and it never imports the product path.  The arithmetic lives in
``spec_oracle.c`` (plain C, fp64, libm ``exp``/``log``, OpenMP over requests);
see that file's header for the rules and the pages each follows.

Near-tie tolerances:
  EPS_ACCEPT  |u - r| (exact) or |p - tau| (relaxed) below this flags the test.
  EPS_SAMPLE  u*Z closer than EPS_SAMPLE*Z to a boundary of the fp64 CDF flags
              the terminal sample.  1e-11: two decades above the oracle's own
              error at V = 128256 (its draws match an extended-precision
              inverse CDF from 1e-13 of Z on) and three above the HIP
              library's measured one (no disagreement down to 1e-14 of Z, with
              uniforms placed next to boundaries).  At V = 128256 it flags
              about 3e-6 of the draws.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = ["build", "load", "OracleResult", "OracleSample", "OracleTrace", "greedy", "exact",
           "relaxed", "tree", "power", "sample", "speculative_generate", "row_stats",
           "terminal_weights", "TerminalWeights",
           "set_threads", "max_threads", "EPS_ACCEPT", "EPS_SAMPLE"]

EPS_ACCEPT = 1e-6
EPS_SAMPLE = 1e-11

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc -O2 (no fast-math) and OpenMP."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        Dd = ctypes.c_double
        lib.oracle_set_threads.argtypes = [I]
        lib.oracle_max_threads.restype = I
        lib.oracle_row_stats.argtypes = [P, I, ctypes.c_long, I, P, P, P]
        lib.oracle_greedy.argtypes = [P, I, P, I, I, I, P, P, P, P, P, P]
        lib.oracle_exact.argtypes = [P, P, I, P, P, I, I, I, Dd, Dd, P, P, P, P, P, P, P]
        lib.oracle_relaxed.argtypes = [P, I, P, P, I, I, I, Dd, I, Dd, Dd, P, P, P, P, P, P, P]
        lib.oracle_sample.argtypes = [P, I, P, ctypes.c_long, I, Dd, P, P, P]
        lib.oracle_power.argtypes = [P, P, I, P, P, I, I, I, Dd, Dd, Dd, P, P, P, P, P, P, P]
        lib.oracle_tree.argtypes = [P, I, P, P, P, I, I, I, P, P, P, P, P, P]
        lib.oracle_terminal_weights.argtypes = [I, P, P, I, P, I, I, I, P, P, P]
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(load().oracle_max_threads())


@dataclass
class OracleResult:
    tokens: np.ndarray          # int32 [B][L], -1 padded
    accept_len: np.ndarray      # int32 [B]
    target_logprob: np.ndarray  # float64 [B][L]
    behavior_logprob: np.ndarray
    status: np.ndarray          # int32 [B]
    flag: np.ndarray            # int32 [B], first near-tie position or -1
    decisions: np.ndarray       # int32 [B]
    path: Optional[np.ndarray] = None  # tree only: node ids [B][N]


def _dt(dtype: str) -> int:
    return BF16 if dtype == "bf16" else F32


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _logits(a, dtype):
    return _c(a, np.uint16 if dtype == "bf16" else np.float32)


def row_stats(x: np.ndarray, dtype: str):
    """(M, g, S) per row of a [..., V] logit array."""
    x = _logits(x, dtype)
    V = x.shape[-1]
    rows = x.size // V
    M = np.empty(rows, np.float64)
    g = np.empty(rows, np.int64)
    S = np.empty(rows, np.float64)
    load().oracle_row_stats(_ptr(x), _dt(dtype), rows, V, _ptr(M), _ptr(g), _ptr(S))
    shp = x.shape[:-1]
    return M.reshape(shp), g.reshape(shp), S.reshape(shp)


def _outs(B, L):
    return (np.empty((B, L), np.int32), np.empty(B, np.int32), np.empty((B, L), np.float64),
            np.empty((B, L), np.float64), np.empty(B, np.int32), np.full(B, -1, np.int32),
            np.empty(B, np.int32))


def greedy(target, tokens, dtype: str) -> OracleResult:
    T = _logits(target, dtype)
    x = _c(tokens, np.int32)
    B, L, V = T.shape
    K = L - 1
    assert x.shape == (B, K)
    tok, ln, tlp, blp, st, fl, dec = _outs(B, L)
    load().oracle_greedy(_ptr(T), _dt(dtype), _ptr(x), B, K, V, _ptr(tok), _ptr(ln), _ptr(tlp),
                         _ptr(blp), _ptr(st), _ptr(dec))
    return OracleResult(tok, ln, tlp, blp, st, fl, dec)


def exact(target, draft, tokens, uniforms, dtype: str, eps_accept: float = EPS_ACCEPT,
          eps_sample: float = EPS_SAMPLE) -> OracleResult:
    T = _logits(target, dtype)
    Dr = _logits(draft, dtype)
    x = _c(tokens, np.int32)
    u = _c(uniforms, np.float32)
    B, L, V = T.shape
    K = L - 1
    assert Dr.shape == (B, K, V) and x.shape == (B, K) and u.shape == (B, L)
    tok, ln, tlp, blp, st, fl, dec = _outs(B, L)
    load().oracle_exact(_ptr(T), _ptr(Dr), _dt(dtype), _ptr(x), _ptr(u), B, K, V,
                        float(eps_accept), float(eps_sample), _ptr(tok), _ptr(ln), _ptr(tlp),
                        _ptr(blp), _ptr(st), _ptr(fl), _ptr(dec))
    return OracleResult(tok, ln, tlp, blp, st, fl, dec)


def relaxed(target, tokens, uniforms, dtype: str, tau: float, top_k: int,
            eps_accept: float = EPS_ACCEPT, eps_sample: float = EPS_SAMPLE) -> OracleResult:
    T = _logits(target, dtype)
    x = _c(tokens, np.int32)
    u = _c(uniforms, np.float32)
    B, L, V = T.shape
    K = L - 1
    assert x.shape == (B, K) and u.shape == (B, L)
    tok, ln, tlp, blp, st, fl, dec = _outs(B, L)
    load().oracle_relaxed(_ptr(T), _dt(dtype), _ptr(x), _ptr(u), B, K, V, float(tau), int(top_k),
                          float(eps_accept), float(eps_sample), _ptr(tok), _ptr(ln), _ptr(tlp),
                          _ptr(blp), _ptr(st), _ptr(fl), _ptr(dec))
    return OracleResult(tok, ln, tlp, blp, st, fl, dec)


def power(target, draft, tokens, uniforms, dtype: str, alpha: float,
          eps_accept: float = EPS_ACCEPT, eps_sample: float = EPS_SAMPLE) -> OracleResult:
    """Power rule: accept iff u_j < min(1, p/q)^alpha; y ~ p_n after a rejection."""
    T = _logits(target, dtype)
    D = _logits(draft, dtype)
    x = _c(tokens, np.int32)
    u = _c(uniforms, np.float32)
    B, L, V = T.shape
    K = L - 1
    assert D.shape == (B, K, V) and x.shape == (B, K) and u.shape == (B, L)
    tok, ln, tlp, blp, st, fl, dec = _outs(B, L)
    load().oracle_power(_ptr(T), _ptr(D), _dt(dtype), _ptr(x), _ptr(u), B, K, V, float(alpha),
                        float(eps_accept), float(eps_sample), _ptr(tok), _ptr(ln), _ptr(tlp),
                        _ptr(blp), _ptr(st), _ptr(fl), _ptr(dec))
    return OracleResult(tok, ln, tlp, blp, st, fl, dec)


@dataclass
class OracleSample:
    """One draw per logit row: token, its log-prob under the row's softmax, and
    a near-boundary flag (u*Z within EPS_SAMPLE*Z of a CDF boundary)."""
    tokens: np.ndarray
    logq: np.ndarray
    flag: np.ndarray


def sample(logits, uniforms, dtype: str, eps_sample: float = EPS_SAMPLE) -> OracleSample:
    """Draft sampler: y = inverse CDF of softmax(row) at the row's uniform.
    logits [..., V]; uniforms with the leading shape of logits."""
    X = _logits(logits, dtype)
    lead, V = X.shape[:-1], X.shape[-1]
    u = _c(uniforms, np.float32)
    assert u.shape == lead
    rows = int(np.prod(lead)) if lead else 1
    tok = np.empty(lead, np.int32)
    lq = np.empty(lead, np.float64)
    fl = np.empty(lead, np.int32)
    load().oracle_sample(_ptr(X), _dt(dtype), _ptr(u), rows, V, float(eps_sample), _ptr(tok),
                         _ptr(lq), _ptr(fl))
    return OracleSample(tok, lq, fl)


@dataclass
class TerminalWeights:
    """The weights a terminal draw inverts: w [B][V] (not normalized), their
    sum Z [B], and for the exact rule whether w is the relu(p - q) residual."""
    w: np.ndarray
    Z: np.ndarray
    residual: np.ndarray


_RULES = {"exact": 0, "target": 1, "sampler": 2}


def terminal_weights(rule: str, target, dtype: str, n=None, draft=None) -> TerminalWeights:
    """Weights of the terminal draw at first-rejection position n[b]:
    rule "exact" (target [B][K+1][V], draft [B][K][V]), "target" (the
    relaxed and power rules' draw from p_n), or "sampler" (target is the
    [rows][V] logits, n unused).  The draw picks the smallest t whose
    running sum of w exceeds u * Z."""
    T = _logits(target, dtype)
    V = T.shape[-1]
    if rule == "sampler":
        B, K = T.size // V, 0
        nn = np.zeros(B, np.int32)
    else:
        B, L, _ = T.shape
        K = L - 1
        nn = _c(n, np.int32)
        assert nn.shape == (B,) and (nn >= 0).all() and (nn <= K).all()
    Dr = _logits(draft, dtype) if draft is not None else None
    if rule == "exact":
        assert Dr is not None and Dr.shape == (B, K, V)
    w = np.empty((B, V), np.float64)
    Z = np.empty(B, np.float64)
    res = np.empty(B, np.int32)
    load().oracle_terminal_weights(_RULES[rule], _ptr(T), None if Dr is None else _ptr(Dr),
                                   _dt(dtype), _ptr(nn), B, K, V, _ptr(w), _ptr(Z), _ptr(res))
    return TerminalWeights(w, Z, res)


def tree(target, node_tok, parents, dtype: str, num_nodes=None) -> OracleResult:
    T = _logits(target, dtype)
    B, N, V = T.shape
    nt = _c(node_tok, np.int32)
    par = _c(parents, np.int32)
    assert nt.shape == (B, N) and par.shape == (B, N)
    nn = None if num_nodes is None else _c(num_nodes, np.int32)
    path = np.empty((B, N), np.int32)
    tok = np.empty((B, N), np.int32)
    ln = np.empty(B, np.int32)
    tlp = np.empty((B, N), np.float64)
    blp = np.empty((B, N), np.float64)
    st = np.empty(B, np.int32)
    load().oracle_tree(_ptr(T), _dt(dtype), _ptr(nt), _ptr(par),
                       None if nn is None else _ptr(nn), B, N, V, _ptr(path), _ptr(tok), _ptr(ln),
                       _ptr(tlp), _ptr(blp), _ptr(st))
    return OracleResult(tok, ln, tlp, blp, st, np.full(B, -1, np.int32),
                        ln.copy(), path=path)


@dataclass
class OracleTrace:
    """A multi-round run: per round and sequence the emitted tokens (-1 padded)
    and the accepted-draft count; per sequence the first round holding a
    flagged near tie (a draft draw or a verification decision), or -1."""
    emitted: np.ndarray     # int32 [rounds][B][K+1]
    accept_len: np.ndarray  # int32 [rounds][B]
    flag_round: np.ndarray  # int32 [B]


def speculative_generate(target_table, draft_table, start, u_draft, u_verify,
                         dtype: str) -> OracleTrace:
    """Speculative sampling over several rounds with toy Markov models, in the
    order of the spec-decode README ("How it works", and generate_speculative
    under "Use it"): each round the draft proposes K tokens one after another
    from its own next-token distribution, the target scores all K+1 positions
    at once, the exact rule accepts a prefix and emits one more token, and the
    next round continues from the last emitted token.  A model's next_dist is
    the row of its table picked by the last token.  Every draw and decision
    is sample() and exact() above; uniforms u_draft[r][b][i] drive draft draw
    i and u_verify[r][b] the verification of round r."""
    T, D = np.asarray(target_table), np.asarray(draft_table)
    rounds, B, K = u_draft.shape
    emitted = np.full((rounds, B, K + 1), -1, np.int32)
    accept_len = np.zeros((rounds, B), np.int32)
    flag_round = np.full(B, -1, np.int32)
    cur = np.asarray(start, np.int32).copy()
    for r in range(rounds):
        prev = [cur]
        hit = np.zeros(B, bool)
        for i in range(K):
            s = sample(D[prev[-1]], u_draft[r, :, i], dtype)
            hit |= s.flag != 0  # 1: the draw sits within the window of a boundary
            prev.append(s.tokens)
        x = np.stack(prev[1:], 1)
        o = exact(T[np.stack(prev, 1)], D[np.stack(prev[:K], 1)], x, u_verify[r], dtype)
        hit |= o.flag >= 0
        flag_round[(flag_round < 0) & hit] = r
        emitted[r] = o.tokens
        accept_len[r] = o.accept_len
        cur = o.tokens[np.arange(B), o.accept_len].astype(np.int32)
    return OracleTrace(emitted, accept_len, flag_round)
