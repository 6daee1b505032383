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

Run statistics follow the README's report: target passes (one per round per
sequence), acceptance rate = accepted drafts / proposed drafts, tokens per
target pass, and the speedup over target-only sampling when one draft step
costs `draft_cost` target passes: tokens / (passes * (1 + K * draft_cost)).
"""
from __future__ import annotations

from typing import NamedTuple

import torch

from . import SpecVerifyError, _check, spec_sample_drafts, spec_verify_exact

__all__ = ["SpeculativeTrace", "generate_speculative", "trace_stats"]


class SpeculativeTrace(NamedTuple):
    emitted: torch.Tensor     # int32 [rounds][B][K+1]: emitted tokens, -1 padded
    accept_len: torch.Tensor  # int32 [rounds][B]: accepted drafts per round


def generate_speculative(target_table: torch.Tensor, draft_table: torch.Tensor,
                         start: torch.Tensor, u_draft: torch.Tensor,
                         u_verify: torch.Tensor) -> SpeculativeTrace:
    """target_table, draft_table [V][V] logits (row s: the next token after s,
    bfloat16 or float32, one dtype); start int32 [B]; u_draft float32
    [rounds][B][K] and u_verify float32 [rounds][B][K+1] uniforms in [0,1)."""
    P = _check(target_table, "target_table")
    if P.dim() != 2 or P.shape[0] != P.shape[1]:
        raise SpecVerifyError("target_table must be [V][V]")
    V = P.shape[0]
    Q = _check(draft_table, "draft_table", P.dtype, (V, V))
    ud = _check(u_draft, "u_draft", torch.float32)
    rounds, B, K = ud.shape
    uv = _check(u_verify, "u_verify", torch.float32, (rounds, B, K + 1))
    cur = _check(start, "start", torch.int32, (B,)).clone()
    emitted = torch.empty((rounds, B, K + 1), dtype=torch.int32, device=P.device)
    accept = torch.empty((rounds, B), dtype=torch.int32, device=P.device)
    rows = torch.arange(B, device=P.device)
    for r in range(rounds):
        prev = [cur]
        for i in range(K):
            d = spec_sample_drafts(Q[prev[-1].long()], ud[r, :, i].contiguous(), logprobs=False)
            prev.append(d.tokens)
        idx = torch.stack(prev, 1).long()
        x = torch.stack(prev[1:], 1)
        res = spec_verify_exact(P[idx], Q[idx[:, :K]], x, uv[r].contiguous(), logprobs=False)
        emitted[r] = res.tokens
        accept[r] = res.accept_len
        cur = res.tokens[rows, res.accept_len.long()].contiguous()
    return SpeculativeTrace(emitted, accept)


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
