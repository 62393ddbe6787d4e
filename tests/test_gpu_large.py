"""GPU parity past 32-bit byte offsets: tensors of more than 4 GB in one call.

70000 tokens routed top-1 to two experts with H = 256 and I = 16384: the saved
gate/up output and dGU are 70000 x 64 KB (4.6 GB), and the big expert's token
segment alone spans 4.58 GB of dGU, so the BF16 weight gradient walks one
segment across the 4 GB mark.

The workload is built so that the oracle stays small: 200 distinct tokens
(seeded as every other workload here), of which the first 100 go to expert 1
and the other 100 to expert 0.  The big call repeats the first 100 tokens 699
times each (tokens 0 .. 69899, token t a copy of distinct token t % 100, all to
expert 1) and ends with the other 100 once (tokens 69900 .. 69999, expert 0).
  * out, dX and dprob of a token depend on that token alone (MXFP8 included: its
    row blocks lie along H, I and 2I of the token), so every row is compared with
    the oracle's row of its distinct token;
  * expert 0's dW sees the same 100 tokens in the same order in both calls;
  * expert 1's BF16 dW is a sum over its tokens, so it is exactly 699 times the
    oracle's dW of the 100 distinct tokens (its MXFP8 dW is not compared: the
    32-token blocks along the segment hold different tokens in the two calls).
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_TOL, MXFP8_TOL, cfg_small, gpu, log, need_gpu, to_np
from moe_inputs import make_inputs
from oracle import mlp

N_DISTINCT, N_SMALL, REPEAT = 100, 100, 699
T_BIG = N_DISTINCT * REPEAT + N_SMALL
H, I = 256, 16384


def _workload():
    cfg_d = cfg_small(T=N_DISTINCT + N_SMALL, H=H, I=I, E=2, k=1)
    idx_d = np.concatenate([np.ones(N_DISTINCT), np.zeros(N_SMALL)]).astype(np.int32)[:, None]
    g = np.random.default_rng(11)
    pr_d = g.uniform(0.2, 1.0, (N_DISTINCT + N_SMALL, 1)).astype(np.float32)
    inp = make_inputs(cfg_d, topk_idx=idx_d, topk_prob=pr_d, with_dy=True)
    src = np.concatenate([np.arange(N_DISTINCT * REPEAT) % N_DISTINCT, N_DISTINCT + np.arange(N_SMALL)])
    s = torch.from_numpy(src)
    dev = torch.device("cuda")
    big = dict(x=inp.x[s].to(dev), idx=torch.from_numpy(idx_d[src]).to(dev),
               prob=torch.from_numpy(pr_d[src]).to(dev), dy=inp.dy[s].to(dev),
               w1=inp.w1.to(dev), w2=inp.w2.to(dev))
    return inp, src, big


@gpu
@pytest.mark.timeout(600)
@pytest.mark.parametrize("compute", ["bf16", "mxfp8", "fp8"])
def test_large_forward(compute):
    m = need_gpu()
    log(f"large fwd {compute}: T={T_BIG} H={H} I={I} E=2 top-1")
    inp, src, b = _workload()
    out, _ = m.moe_grouped_mlp_fwd(b["x"], b["idx"], b["prob"], b["w1"], b["w2"], compute)
    torch.cuda.synchronize()
    fw = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, compute, "bf16")
    err = mlp.normwise_rel_err(to_np(out), fw.out[src])
    log(f"  out={err:.2e}")
    assert err < (BF16_TOL if compute == "bf16" else MXFP8_TOL)


@gpu
@pytest.mark.timeout(600)
@pytest.mark.parametrize("compute", ["bf16", "mxfp8"])
def test_large_backward(compute):
    m = need_gpu()
    log(f"large bwd {compute}: T={T_BIG} H={H} I={I} E=2 top-1")
    inp, src, b = _workload()
    out, ctx = m.moe_grouped_mlp_fwd(b["x"], b["idx"], b["prob"], b["w1"], b["w2"], compute,
                                     save_for_backward=True)
    dx, dprob, dw1, dw2 = m.moe_grouped_mlp_bwd(b["dy"], ctx, b["w1"], b["w2"])
    torch.cuda.synchronize()
    fw = mlp.forward(inp.x, inp.topk_idx.numpy(), inp.topk_prob, inp.w1, inp.w2, compute, "bf16")
    bw = mlp.backward(fw, inp.x, inp.dy, inp.w1, inp.w2)
    errs = {
        "out": mlp.normwise_rel_err(to_np(out), fw.out[src]),
        "dx": mlp.normwise_rel_err(to_np(dx), bw.dx[src]),
        "dprob": mlp.normwise_rel_err(to_np(dprob), bw.dprob[src]),
        "dw1[0]": mlp.normwise_rel_err(to_np(dw1[0]), bw.dw1[0]),
        "dw2[0]": mlp.normwise_rel_err(to_np(dw2[0]), bw.dw2[0]),
    }
    if compute == "bf16":
        errs["dw1[1]"] = mlp.normwise_rel_err(to_np(dw1[1]), REPEAT * bw.dw1[1])
        errs["dw2[1]"] = mlp.normwise_rel_err(to_np(dw2[1]), REPEAT * bw.dw2[1])
    log("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    tol = BF16_TOL if compute == "bf16" else MXFP8_TOL
    for k, v in errs.items():
        assert v < tol, (k, v)
