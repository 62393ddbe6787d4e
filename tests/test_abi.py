"""The C ABI on the host: libmoe.so loads, exports every function include/moe.h
declares, and its host-side logic (size queries, argument validation, status
strings, phase names) answers without touching a GPU.

No call here enqueues GPU work: every compute entry point is only called with
arguments that its validation rejects before anything is launched.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "mixture_experts_grouped_permute_amd", "libmoe.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("moe_", "mxfp8_", "fp8_"))))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmoe.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_four_operations():
    names = _declared()
    for n in ("moe_permute", "mxfp8_quantize", "moe_grouped_mlp_fwd", "moe_grouped_mlp_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        getattr(lib, n)


def test_binding_lists_every_declared_symbol():
    from mixture_experts_grouped_permute_amd import _lib
    assert sorted(_lib.EXPORTS) == _declared()


def test_version_status_and_phase_names(lib):
    assert lib.moe_abi_version() == 7
    lib.moe_status_string.restype = ctypes.c_char_p
    for s in range(5):
        assert lib.moe_status_string(s)
    lib.moe_fwd_phase_name.restype = ctypes.c_char_p
    lib.moe_bwd_phase_name.restype = ctypes.c_char_p
    fwd = [lib.moe_fwd_phase_name(i).decode() for i in range(lib.moe_fwd_phase_count())]
    bwd = [lib.moe_bwd_phase_name(i).decode() for i in range(lib.moe_bwd_phase_count())]
    assert "fc1_gateup_swiglu" in fwd and "fc2_down" in fwd and "combine" in fwd
    assert "wgrad_fc1" in bwd and "dgrad_fc2_swiglu_bwd" in bwd
    assert lib.moe_fwd_phase_name(len(fwd)) is None and lib.moe_fwd_phase_name(-1) is None


def test_permute_workspace_grows_with_rows(lib):
    f = lib.moe_permute_workspace_size
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    a, b = f(4096, 2, 8), f(1 << 20, 2, 8)
    assert 0 < a < b


def _fwd_args(**kw):
    from mixture_experts_grouped_permute_amd._lib import FwdArgs
    E = kw.pop("E", 8)
    tab = (ctypes.c_void_p * E)(*([0x1000] * E))
    a = FwdArgs(T=4096, H=4096, I=14336, E=E, k=2, compute=1, io_dtype=1, x=0x1000, topk_idx=0x1000,
                topk_prob=0x1000, w1=tab, w2=tab, out=0x1000, split_sizes=0x1000, offsets=0x1000,
                row_id_map=0x1000, src_index=0x1000, prob_perm=0x1000)
    for k_, v in kw.items():
        setattr(a, k_, v)
    return a, tab


def test_fwd_workspace_query_and_validation(lib):
    from mixture_experts_grouped_permute_amd._lib import MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE
    lib.moe_grouped_mlp_fwd_workspace.restype = ctypes.c_size_t
    a, tab = _fwd_args()
    bf16 = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
    a.compute = 2
    mx = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
    # MXFP8 additionally holds the E4M3 weights (1 byte per weight + scales)
    assert mx > bf16 > 0 and mx - bf16 >= 8 * 3 * 4096 * 14336 // 2
    # no workspace: rejected on the host before any launch
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(a), None) == MOE_ERR_WORKSPACE
    bad = [dict(T=0), dict(k=9), dict(E=0), dict(E=300), dict(x=0), dict(compute=7), dict(io_dtype=2),
           dict(row_id_map=0), dict(saved_gu=0x1000)]
    for kw in bad:
        b, tb = _fwd_args(**kw)
        assert lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(b)) == 0, kw
        assert lib.moe_grouped_mlp_fwd(ctypes.byref(b), None) == MOE_ERR_INVALID_ARG, kw
    # H not a multiple of the MXFP8 GEMM step: valid, but not implemented
    b, tb = _fwd_args(H=4096 + 64, compute=2)
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(b), None) == MOE_ERR_UNSUPPORTED
    # a null weight pointer in the host table
    b, tb = _fwd_args()
    tb[3] = None
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(b), None) == MOE_ERR_INVALID_ARG


def test_quantize_and_permute_validation(lib):
    from mixture_experts_grouped_permute_amd._lib import MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED
    q = lib.mxfp8_quantize
    q.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    p = 0x1000
    assert q(None, 1, 64, 64, 0, None, 0, p, p, None) == MOE_ERR_INVALID_ARG
    assert q(p, 1, 64, 48, 0, None, 0, p, p, None) == MOE_ERR_UNSUPPORTED   # cols % 32 != 0
    assert q(p, 1, 64, 64, 2, None, 0, p, p, None) == MOE_ERR_INVALID_ARG   # no such axis
    assert q(p, 2, 64, 64, 0, None, 0, p, p, None) == MOE_ERR_INVALID_ARG   # input already MXFP8
    pm = lib.moe_permute
    pm.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_size_t, ctypes.c_void_p]
    # k > E
    assert pm(p, 1, 16, 64, p, p, 5, 4, 1, p, None, p, p, p, p, p, p, 1 << 20, None) == MOE_ERR_INVALID_ARG


def test_fwd_cached_weight_validation(lib):
    from mixture_experts_grouped_permute_amd._lib import MOE_ERR_INVALID_ARG
    lib.moe_grouped_mlp_fwd_workspace.restype = ctypes.c_size_t
    a, tab = _fwd_args(compute=2)
    per_call = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
    a.w1q = a.w1s = a.w2q = a.w2s = 0x2000
    cached = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
    # the cached weights are not copied into the workspace
    assert 0 < cached < per_call and per_call - cached >= 8 * 3 * 4096 * 14336
    b, tb = _fwd_args(compute=1)           # BF16 compute: no MXFP8 weights accepted
    b.w1q = b.w1s = b.w2q = b.w2s = 0x2000
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(b), None) == MOE_ERR_INVALID_ARG
    c, tc = _fwd_args(compute=2)           # all four or none
    c.w1q = 0x2000
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(c), None) == MOE_ERR_INVALID_ARG


def test_fp8_forward_and_quantizer_validation(lib):
    from mixture_experts_grouped_permute_amd._lib import (MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
                                                          MOE_ERR_WORKSPACE, MOE_FP8_E4M3)
    lib.moe_grouped_mlp_fwd_workspace.restype = ctypes.c_size_t
    a, tab = _fwd_args(compute=2)
    mx = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
    b, tb = _fwd_args(compute=MOE_FP8_E4M3)
    f8 = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(b))
    # FP8 holds the bf16 X_perm and h ahead of their quantization, but no E8M0 scales
    assert f8 > 0 and f8 > mx - 8 * 3 * 4096 * 14336 // 32
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(b), None) == MOE_ERR_WORKSPACE
    c, tc = _fwd_args(compute=MOE_FP8_E4M3, H=4096 + 64)          # not a multiple of 128
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(c), None) == MOE_ERR_UNSUPPORTED
    d, td = _fwd_args(compute=MOE_FP8_E4M3)                       # forward only
    d.saved_x_perm = d.saved_gu = d.saved_h = 0x3000
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(d), None) == MOE_ERR_UNSUPPORTED
    e, te = _fwd_args(compute=MOE_FP8_E4M3)                       # E8M0 scales are MXFP8's
    e.w1q = e.w1s = e.w2q = e.w2s = 0x2000
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(e), None) == MOE_ERR_INVALID_ARG
    f, tf = _fwd_args(compute=MOE_FP8_E4M3)                       # cached FP8 codes + fp32 scales
    f.w1q = f.w2q = f.w1_scale = f.w2_scale = 0x2000
    cached = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(f))
    assert 0 < cached < f8 and f8 - cached >= 8 * 3 * 4096 * 14336
    f.w1s = 0x2000                                                # mixed with E8M0 scales
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(f), None) == MOE_ERR_INVALID_ARG
    g_, tg = _fwd_args(compute=2)                                 # MXFP8 takes no fp32 scales
    g_.w1q = g_.w1s = g_.w2q = g_.w2s = g_.w1_scale = 0x2000
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(g_), None) == MOE_ERR_INVALID_ARG
    lib.fp8_tensor_quantize_workspace.restype = ctypes.c_size_t
    lib.fp8_tensor_quantize_workspace.argtypes = [ctypes.c_int]
    assert lib.fp8_tensor_quantize_workspace(8) >= 8 * 4 and lib.fp8_tensor_quantize_workspace(0) == 0
    q = lib.fp8_tensor_quantize
    q.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    p = 0x1000
    assert q(None, 1, 64, 64, None, 1, p, p, p, 1 << 20, None) == MOE_ERR_INVALID_ARG
    assert q(p, 1, 64, 60, None, 1, p, p, p, 1 << 20, None) == MOE_ERR_UNSUPPORTED   # cols % 8 != 0
    assert q(p, 1, 64, 64, None, 2, p, p, p, 1 << 20, None) == MOE_ERR_INVALID_ARG   # 2 groups, no offsets
    assert q(p, 2, 64, 64, None, 1, p, p, p, 1 << 20, None) == MOE_ERR_INVALID_ARG   # input already E4M3
    assert q(p, 1, 64, 64, None, 1, p, p, p, 4, None) == MOE_ERR_WORKSPACE


def test_abi4_debug_outputs_and_error_flag_validation(lib):
    from mixture_experts_grouped_permute_amd._lib import MOE_ERR_INVALID_ARG
    lib.moe_grouped_mlp_fwd_workspace.restype = ctypes.c_size_t
    a, tab = _fwd_args(compute=2)
    per_call = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
    a.h_codes, a.h_scales = 0x2000, 0x3000
    # h's codes and scales go to the caller's buffers: R * I * (1 + 1/32) bytes fewer
    own = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
    assert per_call - own >= 8192 * 14336 * 33 // 32
    a.h_f32 = 0x4000
    a.error_flag = 0x5000
    assert lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a)) == own
    b, tb = _fwd_args(compute=2)           # both or neither
    b.h_codes = 0x2000
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(b), None) == MOE_ERR_INVALID_ARG
    c, tc = _fwd_args(compute=1)           # MXFP8 only
    c.h_codes, c.h_scales = 0x2000, 0x3000
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(c), None) == MOE_ERR_INVALID_ARG
    d, td = _fwd_args(compute=1)           # fp32 h is accepted for any compute
    d.h_f32 = 0x4000
    assert lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(d)) > 0


def test_weight_quantizer_validation(lib):
    from mixture_experts_grouped_permute_amd._lib import MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED
    f = lib.mxfp8_quantize_weights
    f.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    p = 0x1000
    tab = (ctypes.c_void_p * 4)(*([p] * 4))
    assert f(tab, 0, 64, 64, 0, None, p, p, None) == MOE_ERR_INVALID_ARG       # no matrices
    assert f(tab, 4, 64, 64, 2, None, p, p, None) == MOE_ERR_INVALID_ARG       # no such axis
    assert f(tab, 4, 64, 48, 0, None, p, p, None) == MOE_ERR_UNSUPPORTED       # cols % 32
    assert f(tab, 4, 48, 64, 1, None, p, p, None) == MOE_ERR_UNSUPPORTED       # rows % 32 along rows
    assert f(tab, 4, 64, 64, 0, None, None, p, None) == MOE_ERR_INVALID_ARG    # no output
    tab[2] = None
    assert f(tab, 4, 64, 64, 0, None, p, p, None) == MOE_ERR_INVALID_ARG       # a null matrix


def test_bwd_cached_transposed_weight_validation(lib):
    from mixture_experts_grouped_permute_amd._lib import BwdArgs, MOE_ERR_INVALID_ARG
    E = 8
    tab = (ctypes.c_void_p * E)(*([0x1000] * E))

    def args(**kw):
        a = BwdArgs(T=4096, H=4096, I=14336, E=E, k=2, compute=2, io_dtype=1, dw_dtype=0, dy=0x1000, w1=tab, w2=tab,
                    split_sizes=0x1000, offsets=0x1000, row_id_map=0x1000, src_index=0x1000, prob_perm=0x1000,
                    saved_x_perm=0x1000, saved_gu=0x1000, saved_h=0x1000, dx=0x1000, dprob=0x1000, dw1=tab, dw2=tab)
        for k_, v in kw.items():
            setattr(a, k_, v)
        return a

    lib.moe_grouped_mlp_bwd_workspace.restype = ctypes.c_size_t
    per_call = lib.moe_grouped_mlp_bwd_workspace(ctypes.byref(args()))
    cached = lib.moe_grouped_mlp_bwd_workspace(ctypes.byref(args(w1tq=0x2000, w1ts=0x2000, w2tq=0x2000, w2ts=0x2000)))
    assert 0 < cached < per_call and per_call - cached >= E * 3 * 4096 * 14336
    assert lib.moe_grouped_mlp_bwd(ctypes.byref(args(w1tq=0x2000)), None) == MOE_ERR_INVALID_ARG
    bf = args(compute=1, w1tq=0x2000, w1ts=0x2000, w2tq=0x2000, w2ts=0x2000)
    assert lib.moe_grouped_mlp_bwd(ctypes.byref(bf), None) == MOE_ERR_INVALID_ARG


def test_bwd_fused_dgu_debug_validation(lib):
    """ABI 5: the MXFP8 backward quantizes dGU in the FC2 dgrad epilogue and keeps no bf16 dGU in its
    workspace; the five debug outputs go all together, MXFP8 only, and replace workspace buffers."""
    from mixture_experts_grouped_permute_amd._lib import BwdArgs, MOE_ERR_INVALID_ARG
    E, T, k, H, I = 8, 4096, 2, 4096, 14336
    R = T * k
    tab = (ctypes.c_void_p * E)(*([0x1000] * E))

    def args(**kw):
        a = BwdArgs(T=T, H=H, I=I, E=E, k=k, compute=2, io_dtype=1, dw_dtype=0, dy=0x1000, w1=tab, w2=tab,
                    split_sizes=0x1000, offsets=0x1000, row_id_map=0x1000, src_index=0x1000, prob_perm=0x1000,
                    saved_x_perm=0x1000, saved_gu=0x1000, saved_h=0x1000, dx=0x1000, dprob=0x1000, dw1=tab, dw2=tab)
        for k_, v in kw.items():
            setattr(a, k_, v)
        return a

    lib.moe_grouped_mlp_bwd_workspace.restype = ctypes.c_size_t
    dbg = dict(dgu_bf16=0x2000, dgu_codes=0x2000, dgu_scales=0x2000, dgu_t_codes=0x2000, dgu_t_scales=0x2000)
    mx = lib.moe_grouped_mlp_bwd_workspace(ctypes.byref(args()))
    bf = lib.moe_grouped_mlp_bwd_workspace(ctypes.byref(args(compute=1)))
    with_dbg = lib.moe_grouped_mlp_bwd_workspace(ctypes.byref(args(**dbg)))
    rp = ((R + 127) // 128 * 128 + 128 * E + 511) // 512 * 512
    # the debug buffers replace the two quantized copies of dGU (row-wise and along tokens)
    assert 0 < with_dbg < mx and mx - with_dbg >= R * 2 * I + 2 * I * rp
    # bf16 dGU lives in the BF16 workspace only
    assert bf > 0
    for name in dbg:
        one = {name: 0x2000}
        assert lib.moe_grouped_mlp_bwd(ctypes.byref(args(**one)), None) == MOE_ERR_INVALID_ARG
    assert lib.moe_grouped_mlp_bwd(ctypes.byref(args(compute=1, **dbg)), None) == MOE_ERR_INVALID_ARG


def test_fwd_transposed_weight_output_validation(lib):
    """ABI 6: the forward's optional transposed-weight outputs go all four together, MXFP8 with
    per-call weight quantization only; the per-expert loop does not offer them."""
    from mixture_experts_grouped_permute_amd._lib import FwdArgs, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED
    E = 8
    tab = (ctypes.c_void_p * E)(*([0x1000] * E))

    def args(**kw):
        a = FwdArgs(T=4096, H=4096, I=14336, E=E, k=2, compute=2, io_dtype=1, x=0x1000, topk_idx=0x1000,
                    topk_prob=0x1000, w1=tab, w2=tab, out=0x1000, split_sizes=0x1000, offsets=0x1000,
                    row_id_map=0x1000, src_index=0x1000, prob_perm=0x1000)
        for k_, v in kw.items():
            setattr(a, k_, v)
        return a

    lib.moe_grouped_mlp_fwd_workspace.restype = ctypes.c_size_t
    wt = dict(w1tq_out=0x2000, w1ts_out=0x2000, w2tq_out=0x2000, w2ts_out=0x2000)
    assert lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(args(**wt))) > 0
    for name in wt:
        assert lib.moe_grouped_mlp_fwd(ctypes.byref(args(**{name: 0x2000})), None) == MOE_ERR_INVALID_ARG
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(args(compute=1, **wt)), None) == MOE_ERR_INVALID_ARG
    cached = dict(w1q=0x3000, w1s=0x3000, w2q=0x3000, w2s=0x3000)
    assert lib.moe_grouped_mlp_fwd(ctypes.byref(args(**wt, **cached)), None) == MOE_ERR_INVALID_ARG
    counts = (ctypes.c_int32 * E)(*([1024] * E))
    assert lib.moe_grouped_mlp_fwd_loop(ctypes.byref(args(**wt)), counts, None) == MOE_ERR_UNSUPPORTED


def test_noalloc_permute_limit_on_host(lib):
    """moe_permute_noalloc refuses problems beyond its fixed scratch before any HIP call."""
    from mixture_experts_grouped_permute_amd._lib import MOE_ERR_UNSUPPORTED, MOE_ERR_INVALID_ARG, NOALLOC_SCRATCH_BYTES
    lib.moe_permute_workspace_size.restype = ctypes.c_size_t
    lib.moe_permute_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    assert lib.moe_permute_workspace_size(130752, 2, 256) <= NOALLOC_SCRATCH_BYTES
    assert lib.moe_permute_workspace_size(130753, 2, 256) > NOALLOC_SCRATCH_BYTES
    f = lib.moe_permute_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 9
    p = 0x1000
    assert f(None, 1, 130753, 0, p, None, 2, 256, 1, None, None, p, p, p, p, None, None, None) == MOE_ERR_UNSUPPORTED
    assert f(None, 1, 16, 0, p, None, 5, 4, 1, None, None, p, p, p, p, None, None, None) == MOE_ERR_INVALID_ARG


def test_tile_stats_diagnostic_on_host(lib):
    """moe_set_tile_stats: 6 GEMM slots of 256 x 4 waves x 4 words; a short buffer is refused
    before anything is recorded, and NULL (off) is always accepted."""
    from mixture_experts_grouped_permute_amd._lib import MOE_ERR_INVALID_ARG, TILE_STAT_SLOTS
    lib.moe_tile_stats_bytes.restype = ctypes.c_size_t
    lib.moe_set_tile_stats.restype = ctypes.c_int
    lib.moe_set_tile_stats.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    need = lib.moe_tile_stats_bytes()
    assert need == len(TILE_STAT_SLOTS) * 256 * 4 * 4 * 4
    assert lib.moe_set_tile_stats(0x1000, need - 4) == MOE_ERR_INVALID_ARG
    assert lib.moe_set_tile_stats(None, 0) == 0


def test_mfma_probe_rejects_bad_arguments_on_host(lib):
    """moe_mfma_probe: bad kind, iteration count or buffer is refused before any launch."""
    from mixture_experts_grouped_permute_amd._lib import MOE_ERR_INVALID_ARG
    lib.moe_probe_workgroups.restype = ctypes.c_int
    lib.moe_mfma_probe.restype = ctypes.c_int
    lib.moe_mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.moe_probe_workgroups() == 256
    assert lib.moe_mfma_probe(5, 10, 0x1000, 0x1000, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_mfma_probe(-1, 10, 0x1000, 0x1000, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_mfma_probe(0, 0, 0x1000, 0x1000, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_mfma_probe(0, (1 << 20) + 1, 0x1000, 0x1000, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_mfma_probe(2, 10, None, 0x1000, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_mfma_probe(2, 10, 0x1000, None, None) == MOE_ERR_INVALID_ARG


def test_load_probe_rejects_bad_arguments_on_host(lib):
    """moe_load_probe: bad pattern, stage count, pointer or a short buffer is refused before any
    launch."""
    from mixture_experts_grouped_permute_amd._lib import MOE_ERR_INVALID_ARG
    lib.moe_load_probe_bytes.restype = ctypes.c_size_t
    lib.moe_load_probe.restype = ctypes.c_int
    lib.moe_load_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_void_p]
    need = lib.moe_load_probe_bytes()
    assert need == 512 << 20
    p = 0x1000
    assert lib.moe_load_probe(4, 16, p, need, p, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_load_probe(-1, 16, p, need, p, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_load_probe(0, 0, p, need, p, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_load_probe(0, (1 << 16) + 1, p, need, p, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_load_probe(0, 16, None, need, p, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_load_probe(0, 16, p, need - 1, p, None) == MOE_ERR_INVALID_ARG
    assert lib.moe_load_probe(0, 16, p, need, None, None) == MOE_ERR_INVALID_ARG
