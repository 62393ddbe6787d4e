"""The per-wave cycle-count diagnostic of the grouped GEMMs (moe_set_tile_stats): turning it on
leaves every output bit-identical, and each recording launch fills its slot -- every wave's
words carry the tag, and the work items of the four waves of a workgroup agree."""
import numpy as np
import pytest
import torch

from gpu_util import cfg_small, gpu, log, need_gpu
from moe_inputs import make_inputs


@gpu
@pytest.mark.parametrize("compute", ["bf16", "mxfp8"])
def test_tile_stats_leave_outputs_unchanged(compute):
    m = need_gpu()
    cfg = cfg_small(T=700, H=512, I=768, E=4, k=2)
    inp = make_inputs(cfg, with_dy=True)
    d = inp.to("cuda")

    def run():
        out, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, compute, save_for_backward=True)
        grads = m.moe_grouped_mlp_bwd(d.dy, ctx, d.w1, d.w2)
        torch.cuda.synchronize()
        return [out] + [g for g in grads]

    ref = run()
    buf = m.tile_stats_new("cuda")
    m.set_tile_stats(buf)
    try:
        got = run()
    finally:
        m.set_tile_stats(None)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    w = buf.view(6, 256, 4, 4).cpu().numpy().astype(np.uint32)
    assert (w[..., 3] == 0x7153).all()
    items = w[..., 2]
    assert (items == items[:, :, :1]).all()          # the 4 waves of a workgroup take the same items
    assert (items.sum(axis=(1, 2)) > 0).all()
    summary = m.tile_stats_summary(buf)
    log(f"{compute}: " + ", ".join(f"{k} {v['main_cycles_per_item']}+{v['epilogue_cycles_per_item']}" for k, v in summary.items()))
    assert set(summary) == {"fc1", "fc2", "dgrad_fc2", "wgrad_fc2", "dgrad_fc1", "wgrad_fc1"}
