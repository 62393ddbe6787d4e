"""Shared helpers for the GPU parity tests (imported by tests only)."""
import os
import sys

import numpy as np
import pytest
import torch

from moe_inputs import get_config, make_inputs
from moe_inputs.generate import routing_with_counts

gpu = pytest.mark.gpu

BF16_TOL = 5e-3     # normwise relative error, BF16 path
MXFP8_TOL = 2e-2    # normwise relative error, MXFP8 path


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_grouped_permute_amd as m
    m.load()   # raises loudly when libmoe.so is missing
    return m


def log(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def cfg_small(T, H, I, E, k, precision="bf16", x_dtype="bf16", seed=7):
    return get_config(1).with_(T=T, H=H, I=I, E=E, k=k, precision=precision, x_dtype=x_dtype, seed=seed)


def inputs_with_counts(cfg, counts, seed=3):
    idx, pr = routing_with_counts(counts, cfg.T, cfg.k, seed)
    return make_inputs(cfg, topk_idx=idx, topk_prob=pr)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.to(torch.float64).numpy()
    return t.numpy()
