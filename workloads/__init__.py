"""Seeded synthetic MoE routing workloads.

This module only draws inputs: routing ids, routing weights, token rows and
upstream gradients. It holds none of the arithmetic of prepare, dispatch,
combine or their backward ops, and both the CPU oracle (under ``oracle/``) and
the HIP library are fed from it.

Shapes and distributions follow the MoE models that the expert-parallel pages
name as their targets ("Expert-parallel implementations for
ep_dispatch_experts: all-reduce at inference, all-to-all in training",
validation section; "[PyTorch] Expert Parallelism: PyTorch wrapper + autograd
ops with symm-mem zero-copy", summary: bf16 payloads, int64 routing ids).

Every draw comes from ``numpy.random.SeedSequence(seed_base + config_index)``
spawned into independent streams for routing, tokens, weights and gradients,
so a (config, seed) pair always yields the same bytes.

bf16 tensors are returned as ``numpy.uint16`` bit patterns. The fp32 -> bf16
step uses PyTorch's own CPU conversion (a library routine), so no rounding code
of this project is involved in making inputs.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

MASKED = -1  # routing id of a route that goes to no local expert


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    index: int          # position in CONFIGS, selects the seed stream
    T: int              # tokens
    H: int              # hidden size (bf16 elements per row)
    E: int              # local experts seen by prepare
    K: int              # routes per token (top-k)
    A: int              # per-expert segment alignment, in rows
    routing: str        # uniform | zipf | group_limited
    weights: str        # softmax | sigmoid
    experts: str        # identity | per_expert_scale | weighted
    local_slice: Optional[int] = None   # keep ids < local_slice, others -> -1
    hot_fraction: Optional[float] = None  # force expert 0 into this share of tokens
    global_E: Optional[int] = None      # experts the router picks from


CONFIGS = {
    "tiny": Config("tiny", 0, 256, 512, 8, 2, 16, "uniform", "softmax", "identity"),
    "mixtral": Config("mixtral", 1, 16384, 4096, 8, 2, 128, "uniform", "softmax",
                      "per_expert_scale"),
    "qwen3": Config("qwen3", 2, 8192, 2048, 128, 8, 128, "zipf", "softmax", "weighted"),
    "dsv3": Config("dsv3", 3, 4096, 7168, 256, 8, 128, "group_limited", "sigmoid",
                   "weighted"),
    "masked": Config("masked", 4, 32768, 7168, 32, 8, 128, "group_limited", "sigmoid",
                     "weighted", local_slice=32, global_E=256),
    "masked_hot": Config("masked_hot", 5, 32768, 7168, 32, 8, 128, "group_limited",
                         "sigmoid", "weighted", local_slice=32, hot_fraction=0.86,
                         global_E=256),
}

SEED_BASE = 1000


def scaled(cfg: Config, T: Optional[int] = None, H: Optional[int] = None,
           name: Optional[str] = None) -> Config:
    """The same routing recipe at another token count or hidden size."""
    return dataclasses.replace(cfg, T=cfg.T if T is None else T,
                               H=cfg.H if H is None else H,
                               name=name or cfg.name)


def _streams(cfg: Config, seed: int):
    ss = np.random.SeedSequence(SEED_BASE + cfg.index + 7919 * seed)
    routing, tokens, weights, grads, extra = ss.spawn(5)
    return (np.random.default_rng(routing), np.random.default_rng(tokens),
            np.random.default_rng(weights), np.random.default_rng(grads),
            np.random.default_rng(extra))


def _topk_desc(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row, best first."""
    part = np.argpartition(-scores, k - 1, axis=1)[:, :k]
    order = np.argsort(-np.take_along_axis(scores, part, axis=1), axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1)


def _route_uniform(rng, T, E, K):
    keys = rng.random((T, E))
    return _topk_desc(keys, K), None


def _route_zipf(rng, T, E, K, s=1.1):
    # Popularity p_e proportional to (e+1)^-s (expert 0 hottest). K distinct
    # picks drawn without replacement proportionally to p, via Gumbel-top-K.
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    g = rng.gumbel(size=(T, E))
    return _topk_desc(logp[None, :] + g, K), None


def _route_group_limited(rng, T, E, K, groups=8, top_groups=4):
    # N(0,1) affinity scores; group score = max over the group's experts;
    # keep the best top_groups groups, then the K best experts inside them.
    scores = rng.standard_normal((T, E)).astype(np.float32)
    gsize = E // groups
    gscore = scores.reshape(T, groups, gsize).max(axis=2)
    keep = _topk_desc(gscore, top_groups)
    mask = np.zeros((T, groups), dtype=bool)
    np.put_along_axis(mask, keep, True, axis=1)
    masked_scores = np.where(np.repeat(mask, gsize, axis=1), scores, -np.inf)
    idx = _topk_desc(masked_scores, K)
    return idx, np.take_along_axis(scores, idx, axis=1)


def _bf16_bits(f32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact) for building expert outputs."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.float().numpy()


def randn_bf16(rng, shape) -> np.ndarray:
    return _bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@dataclasses.dataclass
class Routing:
    topk_idx: np.ndarray       # int64 [T, K]; -1 = masked
    topk_weights: np.ndarray   # float32 [T, K]
    hot_share: Optional[float] = None  # realised share of valid routes on expert 0


def make_routing(cfg: Config, seed: int = 0) -> Routing:
    rng_r, _, rng_w, _, rng_x = _streams(cfg, seed)
    T, K = cfg.T, cfg.K
    E_pick = cfg.global_E or cfg.E
    scores = None
    if cfg.routing == "uniform":
        idx, _ = _route_uniform(rng_r, T, E_pick, K)
    elif cfg.routing == "zipf":
        idx, _ = _route_zipf(rng_r, T, E_pick, K)
    elif cfg.routing == "group_limited":
        idx, scores = _route_group_limited(rng_r, T, E_pick, K)
    else:
        raise ValueError(cfg.routing)
    idx = idx.astype(np.int64)
    if cfg.hot_fraction is not None:
        # Expert 0 joins the top-K of a Bernoulli(hot_fraction) subset of
        # tokens, replacing the lowest-ranked pick when it is not already there.
        pick = rng_x.random(T) < cfg.hot_fraction
        has0 = (idx == 0).any(axis=1)
        rows = np.nonzero(pick & ~has0)[0]
        idx[rows, K - 1] = 0
        if scores is not None:
            scores[rows, K - 1] = np.float32(3.0)
    if cfg.weights == "softmax":
        logits = rng_w.standard_normal((T, K)).astype(np.float32)
        ex = np.exp(logits - logits.max(axis=1, keepdims=True))
        w = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    elif cfg.weights == "sigmoid":
        if scores is None:
            scores = rng_w.standard_normal((T, K)).astype(np.float32)
        sg = 1.0 / (1.0 + np.exp(-scores.astype(np.float64)))
        w = (sg / sg.sum(axis=1, keepdims=True)).astype(np.float32)
    else:
        raise ValueError(cfg.weights)
    hot_share = None
    if cfg.local_slice is not None:
        idx = np.where(idx < cfg.local_slice, idx, MASKED).astype(np.int64)
        valid = idx >= 0
        if cfg.hot_fraction is not None:
            hot_share = float((idx == 0).sum()) / max(1, int(valid.sum()))
    return Routing(np.ascontiguousarray(idx), np.ascontiguousarray(w), hot_share)


def make_tokens(cfg: Config, seed: int = 0) -> np.ndarray:
    """Token rows x, bf16 bits [T, H], drawn N(0,1)."""
    _, rng_x, _, _, _ = _streams(cfg, seed)
    return randn_bf16(rng_x, (cfg.T, cfg.H))


def make_grads(cfg: Config, recv_rows: int, seed: int = 0):
    """Upstream gradients for the backward ops.

    Returns (g_result bf16 [T,H], g_recv bf16 [recv_rows,H], g_recv_w f32 [recv_rows]),
    all N(0,1).
    """
    _, _, _, rng_g, _ = _streams(cfg, seed)
    g_result = randn_bf16(rng_g, (cfg.T, cfg.H))
    g_recv = randn_bf16(rng_g, (recv_rows, cfg.H))
    g_recv_w = rng_g.standard_normal(recv_rows, dtype=np.float32)
    return g_result, g_recv, g_recv_w


def make_expert_rows(cfg: Config, rows: int, seed: int = 0) -> np.ndarray:
    """Generic expert-output rows, bf16 bits [rows, H], drawn N(0,1)."""
    _, _, _, _, rng_e = _streams(cfg, seed + 1)
    return randn_bf16(rng_e, (rows, cfg.H))


def small_int_bf16(rng, shape, bound: int = 16) -> np.ndarray:
    """bf16 bits of integers in [-bound, bound]: sums of a few stay exact."""
    v = rng.integers(-bound, bound + 1, size=shape).astype(np.float32)
    return _bf16_bits(v)


def randn_bf16_torch(shape, seed: int, device="cuda"):
    """N(0,1) bf16 tensor drawn with PyTorch's seeded generator on ``device``.

    Used for the large payloads of full-size runs, where host generation
    would dominate; the same tensor (copied to the host) feeds the oracle."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(SEED_BASE * 1_000_003 + int(seed))
    return torch.randn(tuple(shape), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)
