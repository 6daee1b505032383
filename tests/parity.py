"""Helpers for comparing the HIP library with the fp64 oracle.

Parity rule:
  * accepted counts and emitted tokens are bit-exact, except where the oracle
    flags a near-tie decision: from the flagged position on, that request is
    exempt (tokens before it must still match, and both sides must have
    accepted at least that many drafts);
  * target and behaviour log-probs agree within LOGPROB_TOL absolute on every
    non-exempt emitted position;
  * padding past the emitted length is -1 (tokens) and 0 (log-probs);
  * flagged near-ties stay under 1e-4 of the decisions.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

LOGPROB_TOL = 1e-4
NEAR_TIE_BUDGET = 1e-4
U_REJECT = np.float32(1.0 - 2.0 ** -24)  # the largest float32 below 1: rejects any r < 1 - 6e-8


def dev_logits(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class Tally:
    requests: int = 0
    decisions: int = 0
    flagged: int = 0

    def add(self, other: "Tally"):
        self.requests += other.requests
        self.decisions += other.decisions
        self.flagged += other.flagged

    def within_budget(self) -> bool:
        """Flagged near-ties strictly under NEAR_TIE_BUDGET of the decisions
        (below 1e4 decisions: none at all)."""
        return self.flagged < NEAR_TIE_BUDGET * self.decisions


def compare_chain(res, orc, *, logprobs=True, what="") -> Tally:
    tok = res.tokens.cpu().numpy()
    ln = res.accept_len.cpu().numpy()
    st = res.status.cpu().numpy()
    tlp = res.target_logprob.cpu().numpy() if (logprobs and res.target_logprob is not None) else None
    blp = res.behavior_logprob.cpu().numpy() if (logprobs and res.behavior_logprob is not None) else None
    B, L = tok.shape
    t = Tally(requests=B, decisions=int(orc.decisions.sum()), flagged=int((orc.flag >= 0).sum()))
    for b in range(B):
        f = int(orc.flag[b])
        ctx = f"{what} request {b}: gpu len {ln[b]} tok {tok[b].tolist()} | oracle len " \
              f"{orc.accept_len[b]} tok {orc.tokens[b].tolist()} flag {f}"
        if f >= 0:
            assert ln[b] >= f and orc.accept_len[b] >= f, ctx
            assert (tok[b, :f] == orc.tokens[b, :f]).all(), ctx
            if tlp is not None and f > 0:
                assert np.abs(tlp[b, :f] - orc.target_logprob[b, :f]).max() < LOGPROB_TOL, ctx
            continue
        n = int(orc.accept_len[b])
        assert ln[b] == n, ctx
        assert st[b] == orc.status[b], ctx
        assert (tok[b, : n + 1] == orc.tokens[b, : n + 1]).all(), ctx
        assert (tok[b, n + 1:] == -1).all(), ctx
        if tlp is not None:
            d = np.abs(tlp[b, : n + 1] - orc.target_logprob[b, : n + 1]).max()
            assert d < LOGPROB_TOL, f"{ctx} target logprob diff {d}"
            assert (tlp[b, n + 1:] == 0).all(), ctx
        if blp is not None:
            d = np.abs(blp[b, : n + 1] - orc.behavior_logprob[b, : n + 1]).max()
            assert d < LOGPROB_TOL, f"{ctx} behavior logprob diff {d}"
            assert (blp[b, n + 1:] == 0).all(), ctx
    return t


def compare_tree(res, orc, *, logprobs=True, what=""):
    path = res.path_nodes.cpu().numpy()
    tok = res.tokens.cpu().numpy()
    ln = res.accept_len.cpu().numpy()
    st = res.status.cpu().numpy()
    tlp = res.target_logprob.cpu().numpy() if logprobs else None
    blp = res.behavior_logprob.cpu().numpy() if logprobs else None
    B, N = tok.shape
    for b in range(B):
        d = int(orc.accept_len[b])
        ctx = f"{what} request {b}: gpu path {path[b].tolist()} oracle {orc.path[b].tolist()}"
        assert ln[b] == d, ctx
        assert st[b] == orc.status[b], ctx
        assert (path[b] == orc.path[b]).all(), ctx
        assert (tok[b, : d + 1] == orc.tokens[b, : d + 1]).all(), ctx
        assert (tok[b, d + 1:] == -1).all(), ctx
        if tlp is not None:
            assert np.abs(tlp[b, : d + 1] - orc.target_logprob[b, : d + 1]).max() < LOGPROB_TOL, ctx
            assert (tlp[b, d + 1:] == 0).all() and (blp[b] == 0).all(), ctx


# ----------------------------------------------- uniforms next to boundaries
def near_boundary_uniforms(w, Z, bins, per_bin, rng):
    """Float32 uniforms u lying next to boundaries of the inverse CDF of w:
    boundary t sits at cumsum(w)[t] / Z (the running sum through token t).
    The distance of u*Z from that boundary, relative to Z, falls in each
    [lo, hi) of `bins`; per bin at most `per_bin` picks.  The boundaries are
    taken from an extended-precision running sum, the reference here.
    Returns (u, dist, want): want is the smallest t whose extended-precision
    running sum exceeds u * Z."""
    wl = w.astype(np.longdouble)
    c = np.cumsum(wl)
    Zl = c[-1]
    pos = np.flatnonzero(w > 0)
    beta = c[pos[:-1]] / Zl                      # boundaries between drawn tokens
    u = beta.astype(np.float32)
    dist = (u.astype(np.longdouble) - beta).astype(np.float64)  # u*Z - boundary, / Z
    out = []
    for lo, hi in bins:
        sel = np.flatnonzero((np.abs(dist) >= lo) & (np.abs(dist) < hi) & (u > 0) & (u < 1))
        if sel.size > per_bin:
            sel = rng.choice(sel, per_bin, replace=False)
        for k in sel:
            want = int(np.searchsorted(c, u[k].astype(np.longdouble) * Zl, side="right"))
            out.append((u[k], dist[k], want))
    return out


BINS = [(1e-14, 1e-13), (1e-13, 1e-12), (1e-12, 1e-11), (1e-11, 1e-10), (1e-10, 1e-9),
        (1e-9, 1e-7)]
