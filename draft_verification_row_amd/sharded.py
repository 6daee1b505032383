"""Vocabulary-sharded verification: Python binding of the spec_shard_* calls.

When the output layer is split over G devices by vocabulary columns, shard s
holds columns [s*Vs, (s+1)*Vs) of every logit row (Vs = V / G).  Each shard
streams its own columns once into a small record slot; the slots are
all-gathered; every shard then folds them and decides (greedy, tree), or
decides, sums its columns of the terminal row(s) into a sums slot, and after
a second all-gather the shard whose columns hold the terminal draw writes it
(exact rule).

The ``shard_*`` functions marshal one call each (raw device pointers, torch's
current stream).  ``verify_*_sharded`` run all G shards of one call on one
device, where the gathered buffers are shared and every call writes its own
slot in place, so the exchanges need no copies; on G devices the same calls
run one per device with collectives between the steps.  Every step runs in
the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import List, NamedTuple, Optional, Sequence

import torch

from . import (SpecVerifyError, TreeResult, VerifyResult, _check, _dtype_code, _outs, _ptr,
               _raise, _stream_ptr, load_library)

__all__ = ["shard_record_bytes", "shard_sums_bytes", "shard_workspace_bytes",
           "shard_stats_greedy", "shard_stats_tree", "shard_stats_exact",
           "shard_combine_greedy", "shard_combine_tree", "shard_sweep_exact",
           "shard_sample_exact", "shard_sweep_power", "shard_sample_power",
           "verify_greedy_sharded", "verify_tree_sharded", "verify_exact_sharded",
           "verify_power_sharded", "verify_relaxed_sharded", "shard_values_bytes",
           "shard_values_relaxed", "shard_stats_relaxed", "shard_sweep_relaxed",
           "shard_sample_relaxed", "ShardedExactResult"]


def shard_record_bytes(dtype: torch.dtype, B: int, rows_per_request: int, V: int, G: int) -> int:
    code = 1 if dtype == torch.bfloat16 else 0
    return int(load_library().spec_shard_record_bytes(code, B, rows_per_request, V, G))


def shard_sums_bytes(B: int, V: int, G: int) -> int:
    return int(load_library().spec_shard_sums_bytes(B, V, G))


def shard_workspace_bytes(B: int) -> int:
    return int(load_library().spec_shard_workspace_bytes(B))


def _slot(buf: torch.Tensor, name: str) -> torch.Tensor:
    return _check(buf, name, torch.uint8)


def _shard_logits(T: torch.Tensor, name: str, G: int):
    _check(T, name)
    if T.dim() != 3:
        raise SpecVerifyError(f"{name} must be [B][rows][V/G]")
    return T.shape[0], T.shape[1], T.shape[2] * G


# ------------------------------------------------------------ single calls
def shard_stats_greedy(target_shard, G: int, shard: int, out_record: torch.Tensor, *,
                       logprobs: bool = True):
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    rec = _slot(out_record, "out_record")
    rc = load_library().spec_shard_stats_greedy(
        _ptr(target_shard), _dtype_code(target_shard), B, L - 1, V, G, shard, int(logprobs),
        _ptr(rec), rec.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_stats_greedy")


def shard_stats_tree(target_shard, G: int, shard: int, out_record: torch.Tensor,
                     num_nodes: Optional[torch.Tensor] = None, *, logprobs: bool = True):
    B, N, V = _shard_logits(target_shard, "target_shard", G)
    nn = None if num_nodes is None else _check(num_nodes, "num_nodes", torch.int32, (B,))
    rec = _slot(out_record, "out_record")
    rc = load_library().spec_shard_stats_tree(
        _ptr(target_shard), _dtype_code(target_shard), _ptr(nn), B, N, V, G, shard,
        int(logprobs), _ptr(rec), rec.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_stats_tree")


def shard_stats_exact(target_shard, draft_shard, draft_tokens, G: int, shard: int,
                      out_record: torch.Tensor):
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    K = L - 1
    _check(draft_shard, "draft_shard", target_shard.dtype, (B, K, V // G))
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    rec = _slot(out_record, "out_record")
    rc = load_library().spec_shard_stats_exact(
        _ptr(target_shard), _ptr(draft_shard), _dtype_code(target_shard), _ptr(x), B, K, V, G,
        shard, _ptr(rec), rec.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_stats_exact")


def shard_combine_greedy(records: torch.Tensor, dtype: torch.dtype, draft_tokens, V: int, G: int,
                         *, logprobs: bool = True) -> VerifyResult:
    rec = _slot(records, "records")
    x = _check(draft_tokens, "draft_tokens", torch.int32)
    B, K = x.shape
    code = 1 if dtype == torch.bfloat16 else 0
    tok, ln, tlp, blp, st = _outs(B, K + 1, x.device, logprobs)
    rc = load_library().spec_shard_combine_greedy(
        _ptr(rec), rec.numel(), code, _ptr(x), B, K, V, G, _ptr(tok), _ptr(ln), _ptr(tlp), _ptr(blp), _ptr(st),
        _stream_ptr(x.device))
    _raise(rc, "spec_shard_combine_greedy")
    return VerifyResult(tok, ln, tlp, blp, st)


def shard_combine_tree(records: torch.Tensor, dtype: torch.dtype, node_tokens, parents,
                       num_nodes: Optional[torch.Tensor], V: int, G: int, *,
                       logprobs: bool = True) -> TreeResult:
    rec = _slot(records, "records")
    nt = _check(node_tokens, "node_tokens", torch.int32)
    B, N = nt.shape
    par = _check(parents, "parents", torch.int32, (B, N))
    nn = None if num_nodes is None else _check(num_nodes, "num_nodes", torch.int32, (B,))
    code = 1 if dtype == torch.bfloat16 else 0
    tok, ln, tlp, blp, st = _outs(B, N, nt.device, logprobs)
    path = torch.empty((B, N), dtype=torch.int32, device=nt.device)
    rc = load_library().spec_shard_combine_tree(
        _ptr(rec), rec.numel(), code, _ptr(nt), _ptr(par), _ptr(nn), B, N, V, G, _ptr(path), _ptr(tok),
        _ptr(ln), _ptr(tlp), _ptr(blp), _ptr(st), _stream_ptr(nt.device))
    _raise(rc, "spec_shard_combine_tree")
    return TreeResult(path, tok, ln, tlp, blp, st)


def shard_sweep_power(target_shard, draft_shard, records: torch.Tensor, draft_tokens, uniforms,
                      G: int, shard: int, alpha: float, out: VerifyResult, out_sums: torch.Tensor,
                      workspace: torch.Tensor):
    """The power rule's step 2; its records come from shard_stats_exact."""
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    K = L - 1
    _check(draft_shard, "draft_shard", target_shard.dtype, (B, K, V // G))
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    u = _check(uniforms, "uniforms", torch.float32, (B, L))
    rec, sums, ws = _slot(records, "records"), _slot(out_sums, "out_sums"), _slot(workspace, "workspace")
    rc = load_library().spec_shard_sweep_power(
        _ptr(target_shard), _ptr(draft_shard), _dtype_code(target_shard), _ptr(rec), rec.numel(),
        _ptr(x),
        _ptr(u), B, K, V, G, shard, ctypes.c_float(alpha), _ptr(out.tokens), _ptr(out.accept_len),
        _ptr(out.target_logprob), _ptr(out.behavior_logprob), _ptr(out.status), _ptr(sums),
        sums.numel(), _ptr(ws), ws.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_sweep_power")


def shard_sample_power(target_shard, draft_shard, sums: torch.Tensor, uniforms, G: int,
                       shard: int, out: VerifyResult, out_sample_shard: Optional[torch.Tensor],
                       workspace: torch.Tensor):
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    K = L - 1
    _check(draft_shard, "draft_shard", target_shard.dtype, (B, K, V // G))
    u = _check(uniforms, "uniforms", torch.float32, (B, L))
    sm, ws = _slot(sums, "sums"), _slot(workspace, "workspace")
    own = None if out_sample_shard is None else _check(out_sample_shard, "out_sample_shard",
                                                       torch.int32, (B,))
    rc = load_library().spec_shard_sample_power(
        _ptr(target_shard), _ptr(draft_shard), _dtype_code(target_shard), _ptr(sm), sm.numel(),
        _ptr(u), B, K,
        V, G, shard, _ptr(out.tokens), _ptr(out.target_logprob), _ptr(out.behavior_logprob),
        _ptr(own), _ptr(ws), ws.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_sample_power")


def shard_sweep_exact(target_shard, draft_shard, records: torch.Tensor, draft_tokens, uniforms,
                      G: int, shard: int, out: VerifyResult, out_sums: torch.Tensor,
                      workspace: torch.Tensor):
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    K = L - 1
    _check(draft_shard, "draft_shard", target_shard.dtype, (B, K, V // G))
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    u = _check(uniforms, "uniforms", torch.float32, (B, L))
    rec, sums, ws = _slot(records, "records"), _slot(out_sums, "out_sums"), _slot(workspace, "workspace")
    rc = load_library().spec_shard_sweep_exact(
        _ptr(target_shard), _ptr(draft_shard), _dtype_code(target_shard), _ptr(rec), rec.numel(),
        _ptr(x),
        _ptr(u), B, K, V, G, shard, _ptr(out.tokens), _ptr(out.accept_len),
        _ptr(out.target_logprob), _ptr(out.behavior_logprob), _ptr(out.status), _ptr(sums),
        sums.numel(), _ptr(ws), ws.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_sweep_exact")


def shard_sample_exact(target_shard, draft_shard, sums: torch.Tensor, uniforms, G: int,
                       shard: int, out: VerifyResult, out_sample_shard: Optional[torch.Tensor],
                       workspace: torch.Tensor):
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    K = L - 1
    _check(draft_shard, "draft_shard", target_shard.dtype, (B, K, V // G))
    u = _check(uniforms, "uniforms", torch.float32, (B, L))
    sm, ws = _slot(sums, "sums"), _slot(workspace, "workspace")
    own = None if out_sample_shard is None else _check(out_sample_shard, "out_sample_shard",
                                                       torch.int32, (B,))
    rc = load_library().spec_shard_sample_exact(
        _ptr(target_shard), _ptr(draft_shard), _dtype_code(target_shard), _ptr(sm), sm.numel(),
        _ptr(u), B, K,
        V, G, shard, _ptr(out.tokens), _ptr(out.target_logprob), _ptr(out.behavior_logprob),
        _ptr(own), _ptr(ws), ws.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_sample_exact")


# ------------------------------------------------- all shards on one device
def _gathered(nbytes: int, G: int, device) -> torch.Tensor:
    if nbytes == 0:
        raise SpecVerifyError("invalid sizes for a sharded call")
    return torch.empty(G * nbytes, dtype=torch.uint8, device=device)


def _shapes(shards: Sequence[torch.Tensor], name: str):
    if not shards:
        raise SpecVerifyError(f"{name}: no shards")
    B, R, Vs = shards[0].shape
    for t in shards:
        if tuple(t.shape) != (B, R, Vs) or t.dtype != shards[0].dtype:
            raise SpecVerifyError(f"{name}: every shard must be [B][rows][V/G] of one dtype")
    return B, R, Vs * len(shards)


def verify_greedy_sharded(target_shards: Sequence[torch.Tensor], draft_tokens, *,
                          logprobs: bool = True) -> VerifyResult:
    G = len(target_shards)
    B, L, V = _shapes(target_shards, "target_shards")
    dt = target_shards[0].dtype
    slot = shard_record_bytes(dt, B, L, V, G)
    rec = _gathered(slot, G, target_shards[0].device)
    for s, T in enumerate(target_shards):
        shard_stats_greedy(T, G, s, rec[s * slot:(s + 1) * slot], logprobs=logprobs)
    return shard_combine_greedy(rec, dt, draft_tokens, V, G, logprobs=logprobs)


def verify_tree_sharded(target_shards: Sequence[torch.Tensor], node_tokens, parents,
                        num_nodes: Optional[torch.Tensor] = None, *,
                        logprobs: bool = True) -> TreeResult:
    G = len(target_shards)
    B, N, V = _shapes(target_shards, "target_shards")
    dt = target_shards[0].dtype
    slot = shard_record_bytes(dt, B, N, V, G)
    rec = _gathered(slot, G, target_shards[0].device)
    for s, T in enumerate(target_shards):
        shard_stats_tree(T, G, s, rec[s * slot:(s + 1) * slot], num_nodes, logprobs=logprobs)
    return shard_combine_tree(rec, dt, node_tokens, parents, num_nodes, V, G, logprobs=logprobs)


class ShardedExactResult(NamedTuple):
    result: VerifyResult
    sample_shard: torch.Tensor  # int32 [B]: the shard whose columns hold the terminal draw


def verify_exact_sharded(target_shards: Sequence[torch.Tensor],
                         draft_shards: Sequence[torch.Tensor], draft_tokens, uniforms, *,
                         logprobs: bool = True) -> ShardedExactResult:
    return _verify_pq_sharded(target_shards, draft_shards, draft_tokens, uniforms, None, logprobs)


def verify_power_sharded(target_shards: Sequence[torch.Tensor],
                         draft_shards: Sequence[torch.Tensor], draft_tokens, uniforms,
                         alpha: float, *, logprobs: bool = True) -> ShardedExactResult:
    return _verify_pq_sharded(target_shards, draft_shards, draft_tokens, uniforms, alpha, logprobs)


def _verify_pq_sharded(target_shards, draft_shards, draft_tokens, uniforms, alpha, logprobs):
    """The exact rule (alpha None) or the power rule over G shards on one device."""
    G = len(target_shards)
    if len(draft_shards) != G:
        raise SpecVerifyError("one draft shard per target shard")
    B, L, V = _shapes(target_shards, "target_shards")
    K = L - 1
    dt = target_shards[0].dtype
    dev = target_shards[0].device
    slot = shard_record_bytes(dt, B, 2 * K + 1, V, G)
    sslot = shard_sums_bytes(B, V, G)
    rec = _gathered(slot, G, dev)
    sums = _gathered(sslot, G, dev)
    ws = [torch.empty(shard_workspace_bytes(B), dtype=torch.uint8, device=dev) for _ in range(G)]
    out = VerifyResult(*_outs(B, L, dev, logprobs))
    own = torch.empty(B, dtype=torch.int32, device=dev)
    for s in range(G):
        shard_stats_exact(target_shards[s], draft_shards[s], draft_tokens, G, s,
                          rec[s * slot:(s + 1) * slot])
    for s in range(G):
        if alpha is None:
            shard_sweep_exact(target_shards[s], draft_shards[s], rec, draft_tokens, uniforms, G, s,
                              out, sums[s * sslot:(s + 1) * sslot], ws[s])
        else:
            shard_sweep_power(target_shards[s], draft_shards[s], rec, draft_tokens, uniforms, G, s,
                              alpha, out, sums[s * sslot:(s + 1) * sslot], ws[s])
    for s in range(G):
        if alpha is None:
            shard_sample_exact(target_shards[s], draft_shards[s], sums, uniforms, G, s, out, own, ws[s])
        else:
            shard_sample_power(target_shards[s], draft_shards[s], sums, uniforms, G, s, out, own, ws[s])
    return ShardedExactResult(out, own)


# ---------------------------------------------------------------- relaxed
def shard_values_bytes(B: int, K: int) -> int:
    return int(load_library().spec_shard_values_bytes(B, K))


def shard_values_relaxed(target_shard, draft_tokens, G: int, shard: int, out_values: torch.Tensor):
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, L - 1))
    out = _slot(out_values, "out_values")
    rc = load_library().spec_shard_values_relaxed(
        _ptr(target_shard), _dtype_code(target_shard), _ptr(x), B, L - 1, V, G, shard, _ptr(out),
        out.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_values_relaxed")


def shard_stats_relaxed(target_shard, draft_tokens, values: torch.Tensor, G: int, shard: int,
                        out_record: torch.Tensor):
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, L - 1))
    vals, rec = _slot(values, "values"), _slot(out_record, "out_record")
    rc = load_library().spec_shard_stats_relaxed(
        _ptr(target_shard), _dtype_code(target_shard), _ptr(x), _ptr(vals), vals.numel(), B, L - 1,
        V, G, shard,
        _ptr(rec), rec.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_stats_relaxed")


def shard_sweep_relaxed(target_shard, records: torch.Tensor, draft_tokens, uniforms, G: int,
                        shard: int, tau: float, top_k: int, out: VerifyResult,
                        out_sums: torch.Tensor, workspace: torch.Tensor):
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    K = L - 1
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    u = _check(uniforms, "uniforms", torch.float32, (B, L))
    rec, sums, ws = _slot(records, "records"), _slot(out_sums, "out_sums"), _slot(workspace, "workspace")
    rc = load_library().spec_shard_sweep_relaxed(
        _ptr(target_shard), _dtype_code(target_shard), _ptr(rec), rec.numel(), _ptr(x), _ptr(u), B,
        K, V, G,
        shard, ctypes.c_float(tau), int(top_k), _ptr(out.tokens), _ptr(out.accept_len),
        _ptr(out.target_logprob), _ptr(out.behavior_logprob), _ptr(out.status), _ptr(sums),
        sums.numel(), _ptr(ws), ws.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_sweep_relaxed")


def shard_sample_relaxed(target_shard, sums: torch.Tensor, uniforms, G: int, shard: int,
                         out: VerifyResult, out_sample_shard: Optional[torch.Tensor],
                         workspace: torch.Tensor):
    B, L, V = _shard_logits(target_shard, "target_shard", G)
    u = _check(uniforms, "uniforms", torch.float32, (B, L))
    sm, ws = _slot(sums, "sums"), _slot(workspace, "workspace")
    own = None if out_sample_shard is None else _check(out_sample_shard, "out_sample_shard",
                                                       torch.int32, (B,))
    rc = load_library().spec_shard_sample_relaxed(
        _ptr(target_shard), _dtype_code(target_shard), _ptr(sm), sm.numel(), _ptr(u), B, L - 1, V,
        G, shard,
        _ptr(out.tokens), _ptr(out.target_logprob), _ptr(out.behavior_logprob), _ptr(own),
        _ptr(ws), ws.numel(), _stream_ptr(target_shard.device))
    _raise(rc, "spec_shard_sample_relaxed")


def verify_relaxed_sharded(target_shards: Sequence[torch.Tensor], draft_tokens, uniforms,
                           tau: float, top_k: int, *, logprobs: bool = True) -> ShardedExactResult:
    """The relaxed rule over G shards on one device: values, stats, sweep and
    sample steps, each writing its own slot of the shared gathered buffers."""
    G = len(target_shards)
    B, L, V = _shapes(target_shards, "target_shards")
    K = L - 1
    dt = target_shards[0].dtype
    dev = target_shards[0].device
    vslot = shard_values_bytes(B, K)
    slot = shard_record_bytes(dt, B, K + 1, V, G)
    sslot = shard_sums_bytes(B, V, G)
    vals = _gathered(vslot, G, dev)
    rec = _gathered(slot, G, dev)
    sums = _gathered(sslot, G, dev)
    ws = [torch.empty(shard_workspace_bytes(B), dtype=torch.uint8, device=dev) for _ in range(G)]
    out = VerifyResult(*_outs(B, L, dev, logprobs))
    own = torch.empty(B, dtype=torch.int32, device=dev)
    for s in range(G):
        shard_values_relaxed(target_shards[s], draft_tokens, G, s, vals[s * vslot:(s + 1) * vslot])
    for s in range(G):
        shard_stats_relaxed(target_shards[s], draft_tokens, vals, G, s, rec[s * slot:(s + 1) * slot])
    for s in range(G):
        shard_sweep_relaxed(target_shards[s], rec, draft_tokens, uniforms, G, s, tau, top_k, out,
                            sums[s * sslot:(s + 1) * sslot], ws[s])
    for s in range(G):
        shard_sample_relaxed(target_shards[s], sums, uniforms, G, s, out, own, ws[s])
    return ShardedExactResult(out, own)
