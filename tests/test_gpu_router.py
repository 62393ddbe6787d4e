"""GPU parity of the fused router (moe_route_topk, moe_route_permute) against the fp64 router
oracle and the permutation oracle.

Indices and every permutation output are compared bit-exactly; the renormalised
probabilities within 2e-6 absolute (fp32 exp and division against fp64).  Cases: the
Mixtral (8 experts, top-2) and fine-grained (64, top-8) shapes, the widest supported (256,
top-16), one expert, odd k, frequent ties, a masked (-inf) expert, fp32 and bf16 logits, and a
token count that is not a multiple of the 256-token blocks.
"""
import numpy as np
import pytest
import torch

from gpu_util import cfg_small, gpu, log, need_gpu
from moe_inputs import get_config, make_logits
from oracle import numerics as nm
from oracle import router as oracle_router
from oracle.permute import permute as oracle_permute

PROB_TOL = 2e-6


def _logits(case):
    name, T, E, k, kind, dtype = case
    cfg = cfg_small(T=T, H=64, I=64, E=E, k=k, seed=100 + E + k)
    if kind == "zipf":
        cfg = get_config(3).with_(T=T, seed=211)
    lg = make_logits(cfg)
    if kind == "ties":
        lg = np.round(lg * 2) / 2        # few distinct values: many exact ties
    t = torch.from_numpy(lg.astype(np.float32))
    return t.to(dtype) if dtype == torch.bfloat16 else t


CASES = [
    ("mixtral-e8-k2", 3000, 8, 2, "normal", torch.float32),
    ("finegrained-e64-k8", 1500, 64, 8, "normal", torch.bfloat16),
    ("e256-k16", 700, 256, 16, "normal", torch.float32),
    ("one-expert", 513, 1, 1, "normal", torch.float32),
    ("odd-k3", 999, 5, 3, "ties", torch.bfloat16),
    ("ties-e16-k4", 2048, 16, 4, "ties", torch.float32),
    ("zipf-masked-expert", 1111, 8, 2, "zipf", torch.float32),
    # many 64-token blocks, so the permutation's count scan slices each expert's column of the
    # router's block counts over several blocks (256 experts: 256 blocks; 24 experts: 469)
    ("e256-k8-256-blocks", 16384, 256, 8, "normal", torch.float32),
    ("e24-k6-469-blocks", 30000, 24, 6, "normal", torch.bfloat16),
]


@gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_route_topk_matches_oracle(case):
    m = need_gpu()
    name, T, E, k, kind, dtype = case
    log(f"router {name} T={T} E={E} k={k} {dtype}")
    lg = _logits(case)
    idx, prob = m.moe_route_topk(lg.to("cuda"), k)
    torch.cuda.synchronize()
    ref_idx, ref_prob = oracle_router.route_topk(lg, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    err = np.abs(prob.cpu().numpy().astype(np.float64) - ref_prob).max()
    log(f"  max |prob - oracle| = {err:.2e}")
    assert err < PROB_TOL


@gpu
@pytest.mark.parametrize("perm_dtype", ["bf16", "mxfp8"])
@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[4], CASES[6], CASES[7], CASES[8]],
                         ids=["mixtral", "finegrained", "odd-k3", "zipf", "e256-256-blocks", "e24-469-blocks"])
def test_route_permute_matches_oracle(case, perm_dtype):
    m = need_gpu()
    name, T, E, k, kind, dtype = case
    H = 128
    log(f"route+permute {name} {perm_dtype} T={T} E={E} k={k} H={H}")
    lg = _logits(case)
    g = np.random.Generator(np.random.PCG64(17))
    x = torch.from_numpy(g.standard_normal((T, H), dtype=np.float32)).to(torch.bfloat16)
    res = m.moe_route_permute(lg.to("cuda"), x.to("cuda"), k, perm_dtype)
    torch.cuda.synchronize()
    ref_idx, ref_prob = oracle_router.route_topk(lg, k)
    np.testing.assert_array_equal(res["topk_idx"].cpu().numpy(), ref_idx)
    assert np.abs(res["topk_prob"].cpu().numpy() - ref_prob).max() < PROB_TOL
    ref = oracle_permute(ref_idx, E)
    for key in ("split_sizes", "offsets", "row_id_map", "src_index"):
        np.testing.assert_array_equal(res[key].cpu().numpy(), getattr(ref, key))
    # prob_perm is the router's own fp32 output, permuted
    np.testing.assert_array_equal(res["prob_perm"].cpu().numpy(),
                                  res["topk_prob"].cpu().numpy().reshape(-1)[ref.src_index])
    xd = x.to(torch.float64).numpy()
    tok = ref.token_of_row
    if perm_dtype == "bf16":
        np.testing.assert_array_equal(res["x_perm"].cpu().view(torch.int16).numpy(),
                                      x.view(torch.int16).numpy()[tok])
    else:
        c, s = nm.quantize_mxfp8(xd, axis=1)
        np.testing.assert_array_equal(res["x_perm"].cpu().numpy(), c[tok])
        np.testing.assert_array_equal(res["x_perm_scales"].cpu().numpy(), s[tok])


@gpu
def test_route_permute_agrees_with_route_then_permute():
    """The fused histogram gives the same permutation as routing and then permuting."""
    m = need_gpu()
    lg = _logits(("x", 4096, 8, 2, "normal", torch.float32)).to("cuda")
    fused = m.moe_route_permute(lg, None, 2)
    idx, prob = m.moe_route_topk(lg, 2)
    sep = m.moe_permute(None, idx, prob, 8)
    torch.cuda.synchronize()
    for key in ("split_sizes", "offsets", "row_id_map", "src_index", "prob_perm"):
        assert torch.equal(fused[key], sep[key]), key
