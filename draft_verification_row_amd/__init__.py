"""Batched draft-verification sampler for MI355X (gfx950): Python binding.

A thin ctypes layer over ``libspecverify.so`` (the C ABI declared in
``include/spec_verify.h``).  It only marshals arguments: it checks that the
torch tensors are on the GPU, contiguous and of the right dtype and shape,
allocates the outputs and the workspace with torch, and passes
raw device pointers and torch's current HIP stream to the library.  Every
step of verification runs in the library's HIP kernels; there is no CPU
path, and every entry point raises if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

__all__ = ["spec_verify_greedy", "spec_verify_exact", "spec_verify_relaxed", "spec_verify_tree",
           "spec_verify_power", "spec_sample_drafts", "spec_verify_workspace_bytes", "spec_sample_workspace_bytes",
           "VerifyResult", "TreeResult", "SampleResult", "SpecVerifyError",
           "library_path", "load_library", "spec_set_spin_limit", "SPEC_MAX_K", "SPEC_MAX_NODES"]

SPEC_F32, SPEC_BF16 = 0, 1
SPEC_MAX_K = 63
SPEC_MAX_NODES = 64
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libspecverify.so")
_lib = None


class SpecVerifyError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libspecverify.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise SpecVerifyError(
            f"{_LIB_PATH} is missing: build it with `python -m draft_verification_row_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    lib.spec_verify_workspace_bytes.argtypes = [I, I, I]
    lib.spec_verify_workspace_bytes.restype = Z
    lib.spec_status_string.argtypes = [I]
    lib.spec_status_string.restype = ctypes.c_char_p
    lib.spec_verify_greedy.argtypes = [P, I, P, I, I, I, P, P, P, P, P, P, Z, P]
    lib.spec_verify_exact.argtypes = [P, P, I, P, P, I, I, I, P, P, P, P, P, P, Z, P]
    lib.spec_verify_relaxed.argtypes = [P, I, P, P, I, I, I, F, I, P, P, P, P, P, P, Z, P]
    lib.spec_verify_tree.argtypes = [P, I, P, P, P, I, I, I, P, P, P, P, P, P, P, Z, P]
    lib.spec_verify_power.argtypes = [P, P, I, P, P, I, I, I, F, P, P, P, P, P, P, Z, P]
    lib.spec_verify_exact_noalloc.argtypes = [P, P, I, P, P, I, I, I, P, P, P, P, P, P]
    lib.spec_sample_workspace_bytes.argtypes = [I, I]
    lib.spec_sample_workspace_bytes.restype = Z
    lib.spec_sample_drafts.argtypes = [P, I, P, I, I, P, P, P, P, Z, P]
    for fn, n in (("spec_shard_record_bytes", 5), ("spec_shard_sums_bytes", 3),
                  ("spec_shard_workspace_bytes", 1)):
        getattr(lib, fn).argtypes = [I] * n
        getattr(lib, fn).restype = Z
    lib.spec_read_ceiling_out_words.argtypes = [Z]
    lib.spec_read_ceiling_out_words.restype = Z
    lib.spec_read_ceiling.argtypes = [P, Z, P, P]
    lib.spec_read_ceiling.restype = I
    lib.spec_shard_stats_greedy.argtypes = [P, I, I, I, I, I, I, I, P, Z, P]
    lib.spec_shard_stats_tree.argtypes = [P, I, P, I, I, I, I, I, I, P, Z, P]
    lib.spec_shard_stats_exact.argtypes = [P, P, I, P, I, I, I, I, I, P, Z, P]
    lib.spec_shard_combine_greedy.argtypes = [P, Z, I, P, I, I, I, I, P, P, P, P, P, P]
    lib.spec_shard_combine_tree.argtypes = [P, Z, I, P, P, P, I, I, I, I, P, P, P, P, P, P, P]
    lib.spec_shard_sweep_exact.argtypes = [P, P, I, P, Z, P, P, I, I, I, I, I, P, P, P, P, P, P,
                                           Z, P, Z, P]
    lib.spec_shard_sample_exact.argtypes = [P, P, I, P, Z, P, I, I, I, I, I, P, P, P, P, P, Z, P]
    lib.spec_shard_sweep_power.argtypes = [P, P, I, P, Z, P, P, I, I, I, I, I, F, P, P, P, P, P,
                                           P, Z, P, Z, P]
    lib.spec_shard_sample_power.argtypes = [P, P, I, P, Z, P, I, I, I, I, I, P, P, P, P, P, Z, P]
    lib.spec_shard_values_bytes.argtypes = [I, I]
    lib.spec_shard_values_bytes.restype = Z
    lib.spec_shard_values_relaxed.argtypes = [P, I, P, I, I, I, I, I, P, Z, P]
    lib.spec_shard_stats_relaxed.argtypes = [P, I, P, P, Z, I, I, I, I, I, P, Z, P]
    lib.spec_shard_sweep_relaxed.argtypes = [P, I, P, Z, P, P, I, I, I, I, I, F, I, P, P, P, P, P,
                                             P, Z, P, Z, P]
    lib.spec_shard_sample_relaxed.argtypes = [P, I, P, Z, P, I, I, I, I, I, P, P, P, P, P, Z, P]
    lib.spec_set_spin_limit.argtypes = [I]
    lib.spec_set_spin_limit.restype = None
    for fn in ("spec_verify_greedy", "spec_verify_exact", "spec_verify_exact_noalloc",
               "spec_verify_relaxed", "spec_verify_tree",
               "spec_verify_power", "spec_sample_drafts", "spec_shard_stats_greedy",
               "spec_shard_stats_tree", "spec_shard_stats_exact", "spec_shard_combine_greedy",
               "spec_shard_combine_tree", "spec_shard_sweep_exact", "spec_shard_sample_exact",
               "spec_shard_sweep_power", "spec_shard_sample_power", "spec_shard_values_relaxed",
               "spec_shard_stats_relaxed", "spec_shard_sweep_relaxed", "spec_shard_sample_relaxed"):
        getattr(lib, fn).restype = I
    _lib = lib
    return lib


class VerifyResult(NamedTuple):
    tokens: torch.Tensor              # int32 [B][K+1], -1 past accept_len
    accept_len: torch.Tensor          # int32 [B]
    target_logprob: Optional[torch.Tensor]    # float32 [B][K+1] or None
    behavior_logprob: Optional[torch.Tensor]  # float32 [B][K+1] or None
    status: torch.Tensor              # int32 [B]


class TreeResult(NamedTuple):
    path_nodes: torch.Tensor          # int32 [B][N], -1 past accept_len
    tokens: torch.Tensor              # int32 [B][N]
    accept_len: torch.Tensor          # int32 [B]
    target_logprob: Optional[torch.Tensor]
    behavior_logprob: Optional[torch.Tensor]
    status: torch.Tensor


# ---------------------------------------------------------------- helpers
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise SpecVerifyError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _check(t: torch.Tensor, name: str, dtype=None, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise SpecVerifyError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise SpecVerifyError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise SpecVerifyError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise SpecVerifyError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise SpecVerifyError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_workspaces = {}


def spec_set_spin_limit(limit: int) -> None:
    """Testing aid: the bound of the single-launch calls' waits (0: give up at
    the first poll that finds nothing; negative: the default)."""
    load_library().spec_set_spin_limit(int(limit))


def spec_verify_workspace_bytes(B: int, rows_per_request: int, V: int) -> int:
    return int(load_library().spec_verify_workspace_bytes(int(B), int(rows_per_request), int(V)))


def _workspace(device: torch.device, nbytes: int, workspace: Optional[torch.Tensor]):
    """Caller-provided workspace (zero-filled before its first call), or one
    cached per (device, stream), allocated zeroed.  Every call leaves the
    workspace zero-filled again, so calls on one stream may share it."""
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8)
        return workspace
    if nbytes == 0:
        raise SpecVerifyError("invalid sizes for the workspace query")
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _raise(code: int, what: str):
    if code != 0:
        msg = load_library().spec_status_string(code).decode()
        raise SpecVerifyError(f"{what}: status {code} ({msg})")


def _outs(B, L, device, logprobs):
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    tok = torch.empty((B, L), **i32)
    ln = torch.empty(B, **i32)
    st = torch.empty(B, **i32)
    tlp = torch.empty((B, L), **f32) if logprobs else None
    blp = torch.empty((B, L), **f32) if logprobs else None
    return tok, ln, tlp, blp, st


# ----------------------------------------------------------- entry points
def spec_verify_greedy(target_logits: torch.Tensor, draft_tokens: torch.Tensor, *,
                       logprobs: bool = True, workspace: Optional[torch.Tensor] = None
                       ) -> VerifyResult:
    """Greedy chain verification.  target_logits [B][K+1][V], draft_tokens int32 [B][K]."""
    lib = load_library()
    T = _check(target_logits, "target_logits")
    if T.dim() != 3:
        raise SpecVerifyError("target_logits must be [B][K+1][V]")
    B, L, V = T.shape
    K = L - 1
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    dev = T.device
    ws = _workspace(dev, spec_verify_workspace_bytes(B, K + 1, V), workspace)
    tok, ln, tlp, blp, st = _outs(B, L, dev, logprobs)
    rc = lib.spec_verify_greedy(_ptr(T), _dtype_code(T), _ptr(x), B, K, V, _ptr(tok), _ptr(ln),
                                _ptr(tlp), _ptr(blp), _ptr(st), _ptr(ws), ws.numel(),
                                _stream_ptr(dev))
    _raise(rc, "spec_verify_greedy")
    return VerifyResult(tok, ln, tlp, blp, st)


def spec_verify_exact(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                      draft_tokens: torch.Tensor, uniforms: torch.Tensor, *,
                      logprobs: bool = True, workspace: Optional[torch.Tensor] = None
                      ) -> VerifyResult:
    """Exact min(1,p/q) verification with residual resampling.

    target_logits [B][K+1][V], draft_logits [B][K][V] (same dtype),
    draft_tokens int32 [B][K], uniforms float32 [B][K+1].
    """
    lib = load_library()
    T = _check(target_logits, "target_logits")
    if T.dim() != 3:
        raise SpecVerifyError("target_logits must be [B][K+1][V]")
    B, L, V = T.shape
    K = L - 1
    D = _check(draft_logits, "draft_logits", T.dtype, (B, K, V))
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    u = _check(uniforms, "uniforms", torch.float32, (B, L))
    dev = T.device
    ws = _workspace(dev, spec_verify_workspace_bytes(B, 2 * K + 1, V), workspace)
    tok, ln, tlp, blp, st = _outs(B, L, dev, logprobs)
    rc = lib.spec_verify_exact(_ptr(T), _ptr(D), _dtype_code(T), _ptr(x), _ptr(u), B, K, V,
                               _ptr(tok), _ptr(ln), _ptr(tlp), _ptr(blp), _ptr(st), _ptr(ws),
                               ws.numel(), _stream_ptr(dev))
    _raise(rc, "spec_verify_exact")
    return VerifyResult(tok, ln, tlp, blp, st)


def spec_verify_power(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                      draft_tokens: torch.Tensor, uniforms: torch.Tensor, alpha: float, *,
                      logprobs: bool = True, workspace: Optional[torch.Tensor] = None
                      ) -> VerifyResult:
    """Power rule: accept iff u_j < min(1, p/q)^alpha; y ~ p_n after a rejection."""
    lib = load_library()
    T = _check(target_logits, "target_logits")
    if T.dim() != 3:
        raise SpecVerifyError("target_logits must be [B][K+1][V]")
    B, L, V = T.shape
    K = L - 1
    D = _check(draft_logits, "draft_logits", T.dtype, (B, K, V))
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    u = _check(uniforms, "uniforms", torch.float32, (B, L))
    dev = T.device
    ws = _workspace(dev, spec_verify_workspace_bytes(B, 2 * K + 1, V), workspace)
    tok, ln, tlp, blp, st = _outs(B, L, dev, logprobs)
    rc = lib.spec_verify_power(_ptr(T), _ptr(D), _dtype_code(T), _ptr(x), _ptr(u), B, K, V,
                               ctypes.c_float(alpha), _ptr(tok), _ptr(ln), _ptr(tlp), _ptr(blp),
                               _ptr(st), _ptr(ws), ws.numel(), _stream_ptr(dev))
    _raise(rc, "spec_verify_power")
    return VerifyResult(tok, ln, tlp, blp, st)


def spec_verify_relaxed(target_logits: torch.Tensor, draft_tokens: torch.Tensor,
                        uniforms: torch.Tensor, tau: float, top_k: int, *,
                        logprobs: bool = True, workspace: Optional[torch.Tensor] = None
                        ) -> VerifyResult:
    """Relaxed acceptance: p >= tau or rank < top_k.  uniforms float32 [B][K+1] (only [:, K] read)."""
    lib = load_library()
    T = _check(target_logits, "target_logits")
    if T.dim() != 3:
        raise SpecVerifyError("target_logits must be [B][K+1][V]")
    B, L, V = T.shape
    K = L - 1
    x = _check(draft_tokens, "draft_tokens", torch.int32, (B, K))
    u = _check(uniforms, "uniforms", torch.float32, (B, L))
    dev = T.device
    ws = _workspace(dev, spec_verify_workspace_bytes(B, K + 1, V), workspace)
    tok, ln, tlp, blp, st = _outs(B, L, dev, logprobs)
    rc = lib.spec_verify_relaxed(_ptr(T), _dtype_code(T), _ptr(x), _ptr(u), B, K, V,
                                 ctypes.c_float(tau), int(top_k), _ptr(tok), _ptr(ln), _ptr(tlp),
                                 _ptr(blp), _ptr(st), _ptr(ws), ws.numel(), _stream_ptr(dev))
    _raise(rc, "spec_verify_relaxed")
    return VerifyResult(tok, ln, tlp, blp, st)


class SampleResult(NamedTuple):
    tokens: torch.Tensor   # int32 [...]
    logprob: torch.Tensor  # float32 [...], or None
    status: torch.Tensor   # int32 [...]


def spec_sample_workspace_bytes(rows: int, V: int) -> int:
    return int(load_library().spec_sample_workspace_bytes(int(rows), int(V)))


def spec_sample_drafts(logits: torch.Tensor, uniforms: torch.Tensor, *, logprobs: bool = True,
                       workspace: Optional[torch.Tensor] = None) -> SampleResult:
    """Draft-token sampler: one inverse-CDF draw per logit row.  logits
    [..., V]; uniforms float32 with the leading shape of logits."""
    lib = load_library()
    X = _check(logits, "logits")
    if X.dim() < 1:
        raise SpecVerifyError("logits must have a vocabulary dimension")
    lead, V = tuple(X.shape[:-1]), X.shape[-1]
    rows = 1
    for d in lead:
        rows *= d
    u = _check(uniforms, "uniforms", torch.float32, lead)
    dev = X.device
    ws = _workspace(dev, spec_sample_workspace_bytes(rows, V), workspace)
    tok = torch.empty(lead, dtype=torch.int32, device=dev)
    st = torch.empty(lead, dtype=torch.int32, device=dev)
    lq = torch.empty(lead, dtype=torch.float32, device=dev) if logprobs else None
    rc = lib.spec_sample_drafts(_ptr(X), _dtype_code(X), _ptr(u), rows, V, _ptr(tok), _ptr(lq),
                                _ptr(st), _ptr(ws), ws.numel(), _stream_ptr(dev))
    _raise(rc, "spec_sample_drafts")
    return SampleResult(tok, lq, st)


def spec_verify_tree(target_logits: torch.Tensor, node_tokens: torch.Tensor,
                     parents: torch.Tensor, num_nodes: Optional[torch.Tensor] = None, *,
                     logprobs: bool = True, workspace: Optional[torch.Tensor] = None
                     ) -> TreeResult:
    """Greedy tree verification.  target_logits [B][N][V]; node_tokens, parents int32 [B][N]."""
    lib = load_library()
    T = _check(target_logits, "target_logits")
    if T.dim() != 3:
        raise SpecVerifyError("target_logits must be [B][N][V]")
    B, N, V = T.shape
    nt = _check(node_tokens, "node_tokens", torch.int32, (B, N))
    par = _check(parents, "parents", torch.int32, (B, N))
    nn = None if num_nodes is None else _check(num_nodes, "num_nodes", torch.int32, (B,))
    dev = T.device
    ws = _workspace(dev, spec_verify_workspace_bytes(B, N, V), workspace)
    tok, ln, tlp, blp, st = _outs(B, N, dev, logprobs)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    rc = lib.spec_verify_tree(_ptr(T), _dtype_code(T), _ptr(nt), _ptr(par), _ptr(nn), B, N, V,
                              _ptr(path), _ptr(tok), _ptr(ln), _ptr(tlp), _ptr(blp), _ptr(st),
                              _ptr(ws), ws.numel(), _stream_ptr(dev))
    _raise(rc, "spec_verify_tree")
    return TreeResult(path, tok, ln, tlp, blp, st)
