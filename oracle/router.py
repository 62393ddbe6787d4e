"""Top-k router in fp64 -- TEST INFRASTRUCTURE ONLY (the oracle of the fused router).

What is computed (page "BioNeMo Uses Grouped Kernels and MXFP8", Figure 1: a
router sends each token to the top k of its experts and their outputs are
combined as a weighted sum; the router's arithmetic itself is not spelled out on
the pages, so the plain reading is taken):

    p = softmax(logits[t, :])                       over all E experts
    idx[t, :] = the k experts of largest p, in descending p,
                equal p -> lower expert id first
    prob[t, j] = p[idx[t, j]] / sum_j' p[idx[t, j']]   (renormalised over the k)

Softmax is strictly increasing in each logit, so the k largest probabilities
belong to the k largest logits; the selection below ranks the logits
themselves (exact comparisons of the input values, no rounding involved).
"""
from __future__ import annotations

import numpy as np


def route_topk(logits, k: int):
    """logits: [T, E] (float array or CPU tensor).  Returns (idx int32 [T,k], prob float64 [T,k])."""
    if hasattr(logits, "detach"):
        import torch
        lg = logits.detach().to("cpu", torch.float64).numpy()
    else:
        lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # softmax over all experts
    m = lg.max(axis=1, keepdims=True)
    p = np.exp(lg - m)
    p /= p.sum(axis=1, keepdims=True)
    # descending logit, ties -> lower id: a stable sort of -logit
    order = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(p, order, axis=1)
    prob = top / top.sum(axis=1, keepdims=True)
    return order.astype(np.int32), prob


def route_topk_scalar(logits_row, k: int):
    """The same for one token with plain Python loops (small E): repeated selection of the
    largest remaining logit, first occurrence on ties."""
    vals = [float(v) for v in logits_row]
    E = len(vals)
    chosen = []
    for _ in range(k):
        best = -1
        for e in range(E):
            if e in chosen:
                continue
            if best < 0 or vals[e] > vals[best]:
                best = e
        chosen.append(best)
    mx = max(vals)
    den_all = sum(np.exp(v - mx) for v in vals)
    ps = [np.exp(vals[e] - mx) / den_all for e in chosen]
    s = sum(ps)
    return chosen, [q / s for q in ps]
