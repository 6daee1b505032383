"""Multi-round speculative sampling with toy Markov models on the GPU.

The loop of the spec-decode README ("How it works", and generate_speculative
under "Use it"): each round the draft proposes K tokens one after another
from its own next-token distribution, the target scores all K+1 positions at
once, the exact rule accepts a prefix and emits one more token, and the next
round continues from the last emitted token.  A toy model's next_dist(prefix)
is the row of its logit table picked by the last token, so its "forward pass"
is a row lookup (torch indexing); every draw and every decision runs in the
library's kernels: spec_sample_drafts for the K draft tokens,
spec_verify_exact for the verification.

SpeculativeGraph captures every round of one shape in a single HIP graph,
so a run is one graph launch instead of some 35 launches per round from the
host; its replays give the same tokens as the eager loop, bit for bit.

Run statistics follow the README's report: target passes (one per round per
sequence), acceptance rate = accepted drafts / proposed drafts, tokens per
target pass, and the speedup over target-only sampling when one draft step
costs `draft_cost` target passes: tokens / (passes * (1 + K * draft_cost)).
"""
from __future__ import annotations

from typing import NamedTuple

import torch

from . import (SpecVerifyError, _check, spec_sample_drafts, spec_sample_workspace_bytes,
               spec_verify_exact, spec_verify_workspace_bytes)

__all__ = ["SpeculativeTrace", "SpeculativeGraph", "generate_speculative", "trace_stats"]


class SpeculativeTrace(NamedTuple):
    emitted: torch.Tensor     # int32 [rounds][B][K+1]: emitted tokens, -1 padded
    accept_len: torch.Tensor  # int32 [rounds][B]: accepted drafts per round


def _tables(target_table, draft_table):
    P = _check(target_table, "target_table")
    if P.dim() != 2 or P.shape[0] != P.shape[1]:
        raise SpecVerifyError("target_table must be [V][V]")
    V = P.shape[0]
    return P, _check(draft_table, "draft_table", P.dtype, (V, V))


def _workspaces(P, B, K):
    """Workspaces of the round's two library calls."""
    V = P.shape[0]
    u8 = dict(dtype=torch.uint8, device=P.device)
    # zero-filled: the library reads published words as "not written" while
    # they are zero and leaves every byte zero after each call
    return (torch.zeros(spec_sample_workspace_bytes(B, V), **u8),
            torch.zeros(spec_verify_workspace_bytes(B, 2 * K + 1, V), **u8))


def _round(P, Q, cur, udt_r, uv_r, ws, rows, emitted_r, accept_r):
    """One round from the last emitted tokens `cur` int32 [B]: K draft draws
    (udt_r [K][B]: draft step i's uniforms are row i), one exact verification;
    writes the round's outputs and returns the next cur.  rows = arange(B)."""
    K = udt_r.shape[0]
    ws_s, ws_v = ws
    prev = [cur]
    for i in range(K):
        d = spec_sample_drafts(Q[prev[-1]], udt_r[i], logprobs=False, workspace=ws_s)
        prev.append(d.tokens)
    idx = torch.stack(prev, 1)
    res = spec_verify_exact(P[idx], Q[idx[:, :K]], idx[:, 1:].contiguous(), uv_r,
                            logprobs=False, workspace=ws_v)
    emitted_r.copy_(res.tokens)
    accept_r.copy_(res.accept_len)
    return res.tokens[rows, res.accept_len]


def generate_speculative(target_table: torch.Tensor, draft_table: torch.Tensor,
                         start: torch.Tensor, u_draft: torch.Tensor,
                         u_verify: torch.Tensor) -> SpeculativeTrace:
    """target_table, draft_table [V][V] logits (row s: the next token after s,
    bfloat16 or float32, one dtype); start int32 [B]; u_draft float32
    [rounds][B][K] and u_verify float32 [rounds][B][K+1] uniforms in [0,1)."""
    P, Q = _tables(target_table, draft_table)
    ud = _check(u_draft, "u_draft", torch.float32)
    rounds, B, K = ud.shape
    uv = _check(u_verify, "u_verify", torch.float32, (rounds, B, K + 1))
    cur = _check(start, "start", torch.int32, (B,)).clone()
    emitted = torch.empty((rounds, B, K + 1), dtype=torch.int32, device=P.device)
    accept = torch.empty((rounds, B), dtype=torch.int32, device=P.device)
    ws = _workspaces(P, B, K)
    udt = ud.transpose(1, 2).contiguous()
    rows = torch.arange(B, dtype=torch.int32, device=P.device)
    for r in range(rounds):
        cur = _round(P, Q, cur, udt[r], uv[r], ws, rows, emitted[r], accept[r])
    return SpeculativeTrace(emitted, accept)


class SpeculativeGraph:
    """generate_speculative for a fixed (B, K, rounds) on fixed tables,
    captured once in one HIP graph.  run() copies the start tokens and
    uniforms into the graph's input buffers and replays it; the returned
    trace's tensors are the graph's output buffers, overwritten by the next
    run.  Replays are ordered on the stream current at run()."""

    def __init__(self, target_table: torch.Tensor, draft_table: torch.Tensor, B: int, K: int,
                 rounds: int):
        self.P, self.Q = _tables(target_table, draft_table)
        if B < 1 or K < 1 or rounds < 1:
            raise SpecVerifyError("B, K and rounds must be positive")
        dev = self.P.device
        self.B, self.K, self.rounds = B, K, rounds
        self.start = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.u_draft_t = torch.zeros((rounds, K, B), dtype=torch.float32, device=dev)
        self.u_verify = torch.zeros((rounds, B, K + 1), dtype=torch.float32, device=dev)
        self.emitted = torch.empty((rounds, B, K + 1), dtype=torch.int32, device=dev)
        self.accept = torch.empty((rounds, B), dtype=torch.int32, device=dev)
        # Buffers made before the capture and read by the graph belong to the
        # ordinary allocator, so they are held here for the graph's lifetime:
        # freed, their blocks could go to other tensors between replays.
        self._ws = _workspaces(self.P, B, K)
        self._rows = torch.arange(B, dtype=torch.int32, device=dev)
        self.graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(device=dev)
        torch.cuda.synchronize(dev)
        with torch.cuda.graph(self.graph, stream=cap):
            cur = self.start.clone()
            for r in range(rounds):
                cur = _round(self.P, self.Q, cur, self.u_draft_t[r], self.u_verify[r], self._ws,
                             self._rows, self.emitted[r], self.accept[r])
        torch.cuda.synchronize(dev)

    def run(self, start: torch.Tensor, u_draft: torch.Tensor,
            u_verify: torch.Tensor) -> SpeculativeTrace:
        B, K, R = self.B, self.K, self.rounds
        self.start.copy_(_check(start, "start", torch.int32, (B,)))
        self.u_draft_t.copy_(_check(u_draft, "u_draft", torch.float32, (R, B, K)).transpose(1, 2))
        self.u_verify.copy_(_check(u_verify, "u_verify", torch.float32, (R, B, K + 1)))
        self.graph.replay()
        return SpeculativeTrace(self.emitted, self.accept)


def trace_stats(accept_len, K: int, draft_cost: float = 0.1) -> dict:
    """accept_len [rounds][B] (tensor or array) -> the README's run report."""
    a = torch.as_tensor(accept_len).to("cpu", torch.float64)
    passes = a.numel()
    accepted = float(a.sum())
    tokens = accepted + passes
    return {"target_passes": passes, "tokens": int(tokens),
            "acceptance_rate": accepted / (K * passes),
            "tokens_per_target_pass": tokens / passes,
            "draft_cost": draft_cost,
            "speedup": tokens / (passes * (1.0 + K * draft_cost))}
