"""GPU parity of the per-expert-loop forward (moe_grouped_mlp_fwd_loop), the baseline that
grouping replaces: the same layer, against the fp64 oracle (BF16 5e-3, MXFP8 2e-2 normwise) and
against the grouped forward."""
import numpy as np
import pytest
import torch

from gpu_util import BF16_TOL, MXFP8_TOL, cfg_small, gpu, log, need_gpu, to_np
from moe_inputs import get_config, make_inputs
from moe_inputs.generate import routing_with_counts
from oracle import mlp

CASES = [
    ("ragged", cfg_small(T=700, H=256, I=384, E=4, k=2), None),
    ("zeros-first-middle-last", cfg_small(T=400, H=128, I=256, E=8, k=2), [0, 400, 1, 31, 0, 33, 335, 0]),
    ("finegrained-e64-k8", get_config(5).with_(T=512, H=256, I=256, precision="bf16"), None),
]


def _inputs(cfg, counts):
    if counts is None:
        return make_inputs(cfg)
    idx, pr = routing_with_counts(counts, cfg.T, cfg.k, 5)
    return make_inputs(cfg, topk_idx=idx, topk_prob=pr)


@gpu
@pytest.mark.parametrize("name,cfg,counts", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("compute", ["bf16", "mxfp8"])
def test_loop_forward_matches_oracle_and_grouped(name, cfg, counts, compute):
    m = need_gpu()
    if compute == "mxfp8" and (cfg.H % 128 or cfg.I % 128):
        cfg = cfg.with_(I=256)
    log(f"loop fwd {name} {compute} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
    inp = _inputs(cfg, counts)
    d = inp.to("cuda")
    idx = inp.topk_idx.numpy()
    host_counts = np.bincount(idx.ravel(), minlength=cfg.E)
    loop_out, _ = m.moe_grouped_mlp_fwd_loop(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, host_counts, compute)
    grp_out, _ = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, compute)
    torch.cuda.synchronize()
    ref = mlp.forward(inp.x, idx, inp.topk_prob, inp.w1, inp.w2, compute, cfg.x_dtype)
    tol = BF16_TOL if compute == "bf16" else MXFP8_TOL
    err = mlp.normwise_rel_err(to_np(loop_out), ref.out)
    diff = mlp.normwise_rel_err(to_np(loop_out), to_np(grp_out))
    log(f"  loop vs oracle {err:.3e}, loop vs grouped {diff:.3e}")
    assert err < tol
    assert diff < tol


@gpu
def test_loop_rejects_inconsistent_counts():
    m = need_gpu()
    cfg = cfg_small(T=64, H=128, I=128, E=4, k=2)
    d = make_inputs(cfg).to("cuda")
    with pytest.raises(m.MoeError) as ei:
        m.moe_grouped_mlp_fwd_loop(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, [1, 2, 3, 4])   # sum != T*k
    assert ei.value.status == 1
