"""Seeded input generation (numpy PCG64, fixed chunking so the bits do not
depend on the thread count).

Recipe per workload (seed = the workload's seed unless overridden):
  * routing "normal": logits ~ N(0,1) of shape [T,E]; softmax; the k largest
    probabilities in descending order (ties -> lower expert id); renormalised
    over the k chosen; stored as float32.  Slot j holds the j-th largest.
  * routing "zipf": logits = -s*ln(e+1) + Gumbel(0,1), so the top-k draw is a
    Plackett-Luce draw without replacement with weights rank^-s; a forced
    empty expert gets logit -inf.  Probabilities as above from these logits.
  * X ~ N(0,1): float32 kept as float32 for f32 I/O, else rounded to bf16.
  * W1 [E,2I,H], W2 [E,H,I] ~ 0.02*N(0,1), rounded to bf16 (rows [0,I) of
    W1 are the gate projection, rows [I,2I) the up projection).
  * dY ~ N(0,1) rounded to the I/O dtype (backward workloads only).
Rounding float32 -> bf16 here uses torch's own CPU conversion (a library
routine); the layer's arithmetic lives elsewhere.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import MoEConfig

_CHUNK = 1 << 22
_TENSOR_IDS = {"logits": 1, "gumbel": 2, "x": 3, "w1": 4, "w2": 5, "dy": 6, "prob": 7, "perm": 8}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(seed: int, name: str, n: int, kind: str = "normal") -> np.ndarray:
    """n float32 draws; chunk c uses SeedSequence(seed, spawn_key=(tensor, c))."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK
    tid = _TENSOR_IDS[name]

    def work(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid, c))))
        if kind == "normal":
            g.standard_normal(out=out[lo:hi], dtype=np.float32)
        elif kind == "gumbel":
            out[lo:hi] = g.gumbel(size=hi - lo).astype(np.float32)
        elif kind == "uniform":
            g.random(out=out[lo:hi], dtype=np.float32)
        else:
            raise ValueError(kind)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def route_topk(logits: np.ndarray, k: int):
    """softmax over experts, top-k descending (ties -> lower id), renormalise."""
    lg = logits.astype(np.float64)
    m = np.max(lg, axis=1, keepdims=True)
    p = np.exp(lg - m)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(p, order, axis=1)
    top = top / top.sum(axis=1, keepdims=True)
    return order.astype(np.int32), top.astype(np.float32)


def routing_with_counts(counts, T: int, k: int, seed: int):
    """A routing whose per-expert token counts are exactly `counts`.

    The expert ids, each repeated counts[e] times in ascending order, are dealt
    to slot (i // T) of token (i % T); since every count is <= T no token gets
    one expert twice.  Token order is then shuffled and probabilities drawn
    uniformly and normalised per token.
    """
    counts = np.asarray(counts, dtype=np.int64)
    if counts.sum() != T * k or counts.max(initial=0) > T:
        raise ValueError("counts must sum to T*k and each be <= T")
    ids = np.repeat(np.arange(counts.size, dtype=np.int32), counts)
    idx = ids.reshape(k, T).T.copy()
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(_TENSOR_IDS["perm"],))))
    idx = idx[g.permutation(T)]
    pr = g.random((T, k)).astype(np.float64) + 0.05
    pr = np.sort(pr, axis=1)[:, ::-1]
    pr = (pr / pr.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(idx), np.ascontiguousarray(pr)


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor          # [T,H] float32 or bfloat16 (CPU)
    topk_idx: torch.Tensor   # [T,k] int32
    topk_prob: torch.Tensor  # [T,k] float32
    w1: torch.Tensor         # [E,2I,H] bfloat16
    w2: torch.Tensor         # [E,H,I] bfloat16
    dy: Optional[torch.Tensor] = None  # [T,H] I/O dtype

    def to(self, device) -> "MoEInputs":
        mv = lambda t: None if t is None else t.to(device, non_blocking=False).contiguous()
        return MoEInputs(self.cfg, mv(self.x), mv(self.topk_idx), mv(self.topk_prob),
                         mv(self.w1), mv(self.w2), mv(self.dy))


def _bf16(a: np.ndarray, scale: float = 1.0) -> torch.Tensor:
    t = torch.from_numpy(a)
    if scale != 1.0:
        t = t.mul_(scale)
    return t.to(torch.bfloat16)


def make_logits(cfg: MoEConfig, seed: Optional[int] = None) -> np.ndarray:
    """The router logits [T, E] (float64) of a workload's routing recipe."""
    seed = cfg.seed if seed is None else seed
    T, E = cfg.T, cfg.E
    logits = _fill(seed, "logits", T * E).reshape(T, E).astype(np.float64)
    if cfg.routing == "zipf":
        gum = _fill(seed, "gumbel", T * E, kind="gumbel").reshape(T, E).astype(np.float64)
        base = -cfg.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        logits = base[None, :] + gum
    elif cfg.routing != "normal":
        raise ValueError(cfg.routing)
    if cfg.zero_expert is not None:
        logits[:, cfg.zero_expert] = -np.inf
    return logits


def make_routing(cfg: MoEConfig, seed: int):
    return route_topk(make_logits(cfg, seed), cfg.k)


def make_inputs(cfg: MoEConfig, seed: Optional[int] = None, *, topk_idx=None, topk_prob=None,
                with_dy: Optional[bool] = None, weights: bool = True) -> MoEInputs:
    seed = cfg.seed if seed is None else seed
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    if topk_idx is None:
        idx, pr = make_routing(cfg, seed)
    else:
        idx = np.ascontiguousarray(np.asarray(topk_idx, dtype=np.int32))
        pr = np.ascontiguousarray(np.asarray(topk_prob, dtype=np.float32))
    xs = _fill(seed, "x", T * H).reshape(T, H)
    x = torch.from_numpy(xs) if cfg.x_dtype == "f32" else _bf16(xs)
    if weights:
        w1 = _bf16(_fill(seed, "w1", E * 2 * I * H), 0.02).reshape(E, 2 * I, H)
        w2 = _bf16(_fill(seed, "w2", E * H * I), 0.02).reshape(E, H, I)
    else:
        w1 = torch.empty(0, dtype=torch.bfloat16)
        w2 = torch.empty(0, dtype=torch.bfloat16)
    dy = None
    if with_dy or (with_dy is None and cfg.backward):
        d = _fill(seed, "dy", T * H).reshape(T, H)
        dy = torch.from_numpy(d) if cfg.x_dtype == "f32" else _bf16(d)
    return MoEInputs(cfg, x, torch.from_numpy(idx), torch.from_numpy(pr), w1, w2, dy)
