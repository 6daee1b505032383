"""Seeded synthetic inputs for the batched draft-verification sampler.

This module is the only code shared by the fp64 oracle (``oracle/``) and the
HIP path (``draft_verification_row_amd``).  It draws logits, draft tokens,
uniforms and draft trees; it contains none of the verification arithmetic
(no acceptance test, no residual, no inverse CDF, no log-softmax).

Workload shapes follow the speculative-decoding pages:
  * a verify pass scores K drafts plus one bonus slot, so the target holds
    K+1 logit rows per request and the draft holds K rows
    (spec-decode README, "How it works" flowchart; mini-sglang PR #134,
    "Modifications", verify_drafts);
  * randomness is supplied by the caller (spec-decode README, "Use it": the
    generator takes ``rng=np.random.default_rng(0)``), so the uniforms are an
    input here as well;
  * draft trees are EAGLE-style with depth 5 and top-k 4 (nanospec README,
    benchmark section: chain depth 5 / tree depth 5, topk 4).

Draft tokens are drawn from softmax(draft logits) with the Gumbel-max trick
(x = argmax_t(d_t + G_t), G_t i.i.d. standard Gumbel), which samples that
softmax exactly without forming it.

Logit values are stored exactly as the kernels read them: bf16 bit patterns
(``uint16``, round-to-nearest-even from fp32) or float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "bf16_rne", "bf16_to_f32", "ChainInputs", "TreeInputs", "chain_inputs",
    "tiny_exact_v32", "greedy_chain_b8", "exact_b32_k5", "large_b64_k8", "tree_b8_n61", "tree_inputs", "make_tree", "widen",
    "gumbel_max_tokens", "redraw_draft_tokens",
]


# ----------------------------------------------------------------------------
# bf16 storage
# ----------------------------------------------------------------------------
def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(h).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored logits -> float64, exactly."""
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# containers
# ----------------------------------------------------------------------------
@dataclass
class ChainInputs:
    """One batch of chain-verification inputs.

    target   [B][K+1][V]  bf16 bits (uint16) or float32
    draft    [B][K][V]    same dtype, or None when the rule needs no draft
    tokens   [B][K]       int32 draft tokens
    uniforms [B][K+1]     float32 in [0,1); u[b][j] drives test j, u[b][K]
                          drives the terminal sample
    """
    name: str
    dtype: str
    B: int
    K: int
    V: int
    target: np.ndarray
    draft: Optional[np.ndarray]
    tokens: np.ndarray
    uniforms: np.ndarray
    tau: float = 0.1
    top_k: int = 4
    # construction facts (greedy scenarios): expected accepted length per request
    expected_accept_len: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    @property
    def algorithmic_bytes_exact(self) -> int:
        es = 2 if self.dtype == "bf16" else 4
        logits = self.B * (2 * self.K + 1) * self.V * es
        return logits + self.B * self.K * 4 + self.B * (self.K + 1) * 4 + _out_bytes(self.B, self.K + 1)

    @property
    def algorithmic_bytes_greedy(self) -> int:
        es = 2 if self.dtype == "bf16" else 4
        return self.B * (self.K + 1) * self.V * es + self.B * self.K * 4 + _out_bytes_greedy(self.B, self.K + 1)

    @property
    def algorithmic_bytes_relaxed(self) -> int:
        # target rows, draft tokens, the one terminal uniform per request, and
        # the outputs with both log-prob rows
        es = 2 if self.dtype == "bf16" else 4
        return (self.B * (self.K + 1) * self.V * es + self.B * self.K * 4 + self.B * 4 +
                _out_bytes(self.B, self.K + 1))


def _out_bytes(B: int, L: int) -> int:
    # tokens + two log-prob rows (int32/fp32 [B][L]) + accept_len + status
    return B * L * 4 * 3 + B * 4 * 2


def _out_bytes_greedy(B: int, L: int) -> int:
    # tokens + accept_len + status (no log-probs requested)
    return B * L * 4 + B * 4 * 2


@dataclass
class TreeInputs:
    """One batch of tree-verification inputs.

    target    [B][N][V]  logits; row i scores the token that follows node i
    node_tok  [B][N]     token carried by each node (node 0 = root, its token
                         is the last committed token and is never verified)
    parents   [B][N]     parent index, parents[b][0] = -1, parents[b][i] < i
    num_nodes [B]        valid nodes per request
    """
    name: str
    dtype: str
    B: int
    N: int
    V: int
    target: np.ndarray
    node_tok: np.ndarray
    parents: np.ndarray
    num_nodes: np.ndarray
    expected_path: Optional[list] = None  # per request: list of node ids (root excluded)
    expected_bonus: Optional[np.ndarray] = None

    @property
    def algorithmic_bytes(self) -> int:
        # logits, node tokens, parents, node counts; path and token outputs
        # [B][N], accepted length and status (no log-probs requested)
        es = 2 if self.dtype == "bf16" else 4
        B, N = self.B, self.N
        return B * N * self.V * es + B * N * 4 * 2 + B * 4 + B * N * 4 * 2 + B * 4 * 2


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------
def gumbel_max_tokens(logits64: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    """Sample one token per row from softmax(row) by Gumbel-max (exact law)."""
    u = rng.random(logits64.shape)
    # -log(-log u) with u in (0,1); u == 0 has probability 2^-53 per draw
    u = np.maximum(u, np.finfo(np.float64).tiny)
    g = -np.log(-np.log(u))
    return np.argmax(logits64 + g, axis=-1).astype(np.int32)


def redraw_draft_tokens(draft: np.ndarray, dtype: str, rng: np.random.Generator) -> np.ndarray:
    """Fresh draft tokens x ~ softmax(row) for every row of stored draft
    logits [..., V], by Gumbel-max with float32 noise: cheap enough to draw a
    new set of tokens for every round of a long run on the same logits (the
    law differs from the exact one only by the float32 rounding of the
    noise)."""
    d = bf16_to_f32(draft) if dtype == "bf16" else np.asarray(draft, np.float32)
    u = rng.random(d.shape, dtype=np.float32)
    np.maximum(u, np.float32(1e-30), out=u)
    g = -np.log(-np.log(u))
    g += d
    return np.argmax(g, axis=-1).astype(np.int32)


def _rng(seed: int, rnd: int) -> np.random.Generator:
    if rnd == 0:
        return np.random.default_rng(seed)
    return np.random.default_rng([seed, rnd])


def _normal(rng, shape, scale):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def chain_inputs(B: int, K: int, V: int, dtype: str = "bf16", *, seed: int, useed: int,
                 t_scale: float = 3.0, d_noise: float = 0.5, rnd: int = 0,
                 tau: float = 0.1, top_k: int = 4, name: str = "chain",
                 with_draft: bool = True) -> ChainInputs:
    """Target logits t_scale*N(0,1), draft = target + d_noise*N(0,1), x ~ softmax(draft).

    Standard deviations, not variances, are the scales (plainest reading of
    "3*N(0,1)" style notation).
    """
    rng = _rng(seed, rnd)
    t32 = _normal(rng, (B, K + 1, V), t_scale)
    if dtype == "bf16":
        target = bf16_rne(t32)
        tw = bf16_to_f32(target)
    else:
        target = t32
        tw = t32
    draft = None
    if with_draft:
        d32 = (tw[:, :K, :] + _normal(rng, (B, K, V), d_noise)).astype(np.float32)
        if dtype == "bf16":
            draft = bf16_rne(d32)
            dw = bf16_to_f32(draft).astype(np.float64)
        else:
            draft = d32
            dw = d32.astype(np.float64)
        tokens = gumbel_max_tokens(dw, rng)
    else:
        tokens = rng.integers(0, V, size=(B, K), dtype=np.int32)
    urng = _rng(useed, rnd)
    uniforms = urng.random((B, K + 1), dtype=np.float32)
    return ChainInputs(name=name, dtype=dtype, B=B, K=K, V=V, target=target, draft=draft,
                       tokens=tokens, uniforms=uniforms, tau=tau, top_k=top_k)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
def tiny_exact_v32(rounds: int = 1000, seed: int = 1) -> ChainInputs:
    """Tiny exact rejection sampling: B=1, K=4, V=32, fp32, many rounds.

    Target ~ 2*N(0,1), draft = target + 0.7*N(0,1), x ~ softmax(draft).  Each
    round is one B=1 request; the rounds are stacked along the batch axis
    (round r = request r).  Uniforms are default_rng(0).random((rounds,1,5)).
    """
    K, V = 4, 32
    rng = np.random.default_rng(seed)
    t = _normal(rng, (rounds, K + 1, V), 2.0)
    d = (t[:, :K, :] + _normal(rng, (rounds, K, V), 0.7)).astype(np.float32)
    tokens = gumbel_max_tokens(d.astype(np.float64), rng)
    u = np.random.default_rng(0).random((rounds, 1, K + 1), dtype=np.float32).reshape(rounds, K + 1)
    return ChainInputs(name="tiny_exact_v32", dtype="f32", B=rounds, K=K, V=V, target=t, draft=d,
                       tokens=tokens, uniforms=u)


def greedy_chain_b8(seed: int = 2, rnd: int = 0, B: int = 8, K: int = 5, V: int = 128256) -> ChainInputs:
    """Greedy chain verify: bf16 3*N(0,1) target [B][K+1][V].

    For request b, j_b ~ U{0..K}; drafts 0..j_b-1 equal the row argmax (lowest
    index among ties), draft j_b (if j_b < K) is uniform over tokens whose
    logit is strictly below the row max, later drafts are uniform over V.
    By construction the accepted length is j_b and the bonus token is the
    argmax of row j_b.
    """
    rng = _rng(seed, rnd)
    target = bf16_rne(_normal(rng, (B, K + 1, V), 3.0))
    tw = bf16_to_f32(target)
    g = np.argmax(tw, axis=-1)  # first occurrence of the max
    jb = rng.integers(0, K + 1, size=B)
    tokens = rng.integers(0, V, size=(B, K)).astype(np.int32)
    for b in range(B):
        for i in range(int(jb[b])):
            tokens[b, i] = g[b, i]
        if jb[b] < K:
            row = tw[b, jb[b]]
            below = np.flatnonzero(row < row.max())
            tokens[b, jb[b]] = below[rng.integers(0, below.size)]
    urng = _rng(102, rnd)
    uniforms = urng.random((B, K + 1), dtype=np.float32)
    ci = ChainInputs(name="greedy_chain_b8", dtype="bf16", B=B, K=K, V=V, target=target, draft=None,
                     tokens=tokens, uniforms=uniforms, expected_accept_len=jb.astype(np.int32))
    ci.extra["expected_bonus"] = np.array([g[b, jb[b]] for b in range(B)], dtype=np.int32)
    return ci


def exact_b32_k5(seed: int = 3, useed: int = 103, rnd: int = 0, B: int = 32, K: int = 5,
       V: int = 128256) -> ChainInputs:
    """Exact stochastic verify: B=32, K=5, V=128256 bf16; target 3*N(0,1), draft + 0.5*N(0,1)."""
    return chain_inputs(B, K, V, "bf16", seed=seed, useed=useed, t_scale=3.0, d_noise=0.5,
                        rnd=rnd, name="exact_b32_k5")


def large_b64_k8(seed: int = 5, useed: int = 105, rnd: int = 0, B: int = 64, K: int = 8,
       V: int = 151936) -> ChainInputs:
    """Relaxed + exact: B=64, K=8, V=151936 bf16; draft + 0.8*N(0,1); tau=0.1, top-4."""
    return chain_inputs(B, K, V, "bf16", seed=seed, useed=useed, t_scale=3.0, d_noise=0.8,
                        rnd=rnd, tau=0.1, top_k=4, name="large_b64_k8")


# ----------------------------------------------------------------------------
# draft trees
# ----------------------------------------------------------------------------
def make_tree(rng: np.random.Generator, depth: int = 5, topk: int = 4, keep: int = 60):
    """EAGLE-style draft tree (depth 5, top-k 4) pruned to `keep` drafted nodes.

    Depth 1: topk children of the root.  Depth d >= 2: the topk nodes of depth
    d-1 with the highest cumulative score each get topk children whose
    weights are a descending-sorted Dirichlet(1,...,1) draw multiplied into
    the parent's score.  The `keep` highest-scored candidates survive (ties
    broken by creation order); scores fall along every path, so the kept set
    is closed under ancestors.  Nodes are renumbered breadth-first, so every
    parent index is smaller than its child's.

    Returns (parents[keep+1], rank[keep+1]) with node 0 the root; rank[i] is
    the position of node i among its parent's kept children by score
    (0 = highest).
    """
    par = [-1]
    score = [1.0]
    dep = [0]
    frontier = [0]
    for d in range(1, depth + 1):
        if d == 1:
            expand = [0]
        else:
            order = sorted(frontier, key=lambda i: (-score[i], i))
            expand = order[:topk]
        new = []
        for p in expand:
            w = np.sort(rng.dirichlet(np.ones(topk)))[::-1]
            for c in range(topk):
                par.append(p)
                score.append(score[p] * float(w[c]))
                dep.append(d)
                new.append(len(par) - 1)
        frontier = new
    cand = list(range(1, len(par)))
    kept = sorted(cand, key=lambda i: (-score[i], i))[:keep]
    kept_set = set(kept)
    for i in kept:
        assert par[i] == 0 or par[i] in kept_set, "pruned tree is not ancestor-closed"
    order = [0] + sorted(kept, key=lambda i: (dep[i], i))
    new_id = {old: k for k, old in enumerate(order)}
    parents = np.array([-1] + [new_id[par[o]] for o in order[1:]], dtype=np.int32)
    rank = np.zeros(len(order), dtype=np.int32)
    children = {}
    for o in order[1:]:
        children.setdefault(par[o], []).append(o)
    for p, ch in children.items():
        for r, o in enumerate(sorted(ch, key=lambda i: (-score[i], i))):
            rank[new_id[o]] = r
    return parents, rank


def tree_inputs(B: int = 8, V: int = 128256, dtype: str = "bf16", *, seed: int = 4, rnd: int = 0,
                depth: int = 5, topk: int = 4, keep: int = 60, p_match: float = 0.7,
                t_scale: float = 3.0, name: str = "tree") -> TreeInputs:
    """Target logits [B][keep+1][V] at t_scale*N(0,1) plus a seeded tree per request.

    For each parent, its highest-scored kept child carries the argmax of the
    parent's row with probability p_match; every other token is drawn
    uniformly from tokens whose logit is strictly below that row's max, with
    siblings kept distinct.  The expected accepted path follows from this
    construction.
    """
    rng = _rng(seed, rnd)
    N = keep + 1
    t32 = _normal(rng, (B, N, V), t_scale)
    target = bf16_rne(t32) if dtype == "bf16" else t32
    tw = bf16_to_f32(target) if dtype == "bf16" else t32
    g = np.argmax(tw, axis=-1)
    parents = np.zeros((B, N), dtype=np.int32)
    node_tok = np.zeros((B, N), dtype=np.int32)
    paths, bonus = [], np.zeros(B, dtype=np.int32)
    for b in range(B):
        par, rank = make_tree(rng, depth=depth, topk=topk, keep=keep)
        parents[b] = par
        node_tok[b, 0] = rng.integers(0, V)
        kids = {}
        for i in range(1, N):
            kids.setdefault(int(par[i]), []).append(i)
        for p, ch in kids.items():
            row = tw[b, p]
            below = np.flatnonzero(row < row.max())
            used = set()
            for i in sorted(ch, key=lambda i: rank[i]):
                if rank[i] == 0 and rng.random() < p_match:
                    node_tok[b, i] = g[b, p]
                else:
                    while True:
                        t = int(below[rng.integers(0, below.size)])
                        if t not in used:
                            break
                    node_tok[b, i] = t
                used.add(int(node_tok[b, i]))
        # construction: follow the (unique) matching child from the root
        path, cur = [], 0
        while True:
            nxt = [i for i in kids.get(cur, []) if node_tok[b, i] == g[b, cur]]
            if not nxt:
                break
            cur = min(nxt)
            path.append(cur)
        paths.append(path)
        bonus[b] = g[b, cur]
    return TreeInputs(name=name, dtype=dtype, B=B, N=N, V=V, target=target, node_tok=node_tok,
                      parents=parents, num_nodes=np.full(B, N, dtype=np.int32),
                      expected_path=paths, expected_bonus=bonus)


def tree_b8_n61(seed: int = 4, rnd: int = 0, B: int = 8, V: int = 128256) -> TreeInputs:
    """Greedy tree verify: B=8, 61 rows (root + 60 drafted nodes), V=128256 bf16."""
    return tree_inputs(B=B, V=V, dtype="bf16", seed=seed, rnd=rnd, name="tree_b8_n61")


# ----------------------------------------------------------------------------
# toy Markov language models for the multi-round driver
# ----------------------------------------------------------------------------
@dataclass
class MarkovInputs:
    """Toy Markov models (a model is next_dist(prefix) = a table row picked by
    the last token) and the randomness of a multi-round run.

    target    [V][V]          logits of the next token after token s, row s
    draft     [V][V]          the draft model's logits, same layout
    start     [B]             int32 first token of each sequence
    u_draft   [rounds][B][K]  float32 uniforms of the K draft draws per round
    u_verify  [rounds][B][K+1] float32 uniforms of the verification per round
    """
    name: str
    dtype: str
    V: int
    B: int
    K: int
    rounds: int
    target: np.ndarray
    draft: np.ndarray
    start: np.ndarray
    u_draft: np.ndarray
    u_verify: np.ndarray


def markov_inputs(V: int, B: int, K: int, rounds: int, dtype: str = "bf16", *, seed: int,
                  t_scale: float = 2.0, d_noise: float = 0.7, name: str = "markov") -> MarkovInputs:
    """Per state the tiny exact config's recipe: target logits t_scale*N(0,1),
    draft = target + d_noise*N(0,1)."""
    rng = np.random.default_rng(seed)
    t32 = _normal(rng, (V, V), t_scale)
    if dtype == "bf16":
        target = bf16_rne(t32)
        tw = bf16_to_f32(target)
    else:
        target, tw = t32, t32
    d32 = (tw + _normal(rng, (V, V), d_noise)).astype(np.float32)
    draft = bf16_rne(d32) if dtype == "bf16" else d32
    start = rng.integers(0, V, size=B).astype(np.int32)
    u_draft = rng.random((rounds, B, K), dtype=np.float32)
    u_verify = rng.random((rounds, B, K + 1), dtype=np.float32)
    return MarkovInputs(name, dtype, V, B, K, rounds, target, draft, start, u_draft, u_verify)
