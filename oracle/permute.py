"""Token permutation by expert (page "BioNeMo Uses Grouped Kernels and MXFP8",
Grouping fragmented expert workloads: the grouped linear takes a per-expert
token count, split_sizes, and each expert's tokens as one contiguous group;
page "How BioNeMo cuts overhead", Grouping the expert work).

Readings where the pages are silent: within an expert's group, rows are in
ascending order of the flattened (token, slot) index t*k + j (a stable counting
sort), which makes every index unique; split_sizes is int32 with E entries and
offsets is its exclusive prefix sum with E+1 entries.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Permutation:
    split_sizes: np.ndarray   # [E]   int32, tokens routed to each expert
    offsets: np.ndarray       # [E+1] int32, exclusive prefix sum of split_sizes
    row_id_map: np.ndarray    # [T*k] int32, (t*k+j) -> permuted row
    src_index: np.ndarray     # [T*k] int32, permuted row -> t*k+j
    k: int

    @property
    def token_of_row(self) -> np.ndarray:
        return self.src_index // self.k


def permute(topk_idx, E: int) -> Permutation:
    idx = np.asarray(topk_idx)
    if idx.ndim != 2:
        raise ValueError("topk_idx must be [T, k]")
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    src_index = np.argsort(flat, kind="stable")
    split = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(split)])
    row_id_map = np.empty(T * k, dtype=np.int64)
    row_id_map[src_index] = np.arange(T * k)
    return Permutation(split.astype(np.int32), offsets.astype(np.int32),
                       row_id_map.astype(np.int32), src_index.astype(np.int32), k)
