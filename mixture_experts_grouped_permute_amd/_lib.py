"""ctypes binding of libmoe.so: argument marshalling only.

Every step of the layer runs in the library's HIP kernels; this module turns
torch tensors into device pointers and the current HIP stream, allocates the
caller-owned output and workspace buffers with torch, and raises on a non-OK
status.  There is no fallback: if libmoe.so is missing or cannot be loaded,
every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_MXFP8_E4M3, MOE_FP8_E4M3 = 0, 1, 2, 3
MAX_EXPERTS = 256

# every symbol include/moe.h declares
EXPORTS = (
    "moe_abi_version", "moe_status_string", "mxfp8_quantize", "moe_permute_workspace_size", "moe_permute",
    "moe_grouped_mlp_fwd_workspace", "moe_grouped_mlp_fwd", "moe_grouped_mlp_bwd_workspace",
    "moe_grouped_mlp_bwd", "moe_read_device_error", "moe_grouped_mlp_fwd_ex", "moe_fwd_phase_count",
    "moe_fwd_phase_name", "moe_grouped_mlp_bwd_ex", "moe_bwd_phase_count", "moe_bwd_phase_name",
    "moe_route_topk", "moe_route_permute", "moe_grouped_mlp_fwd_loop", "fp8_tensor_quantize_workspace",
    "fp8_tensor_quantize", "mxfp8_quantize_weights", "moe_permute_noalloc", "moe_tile_stats_bytes",
    "moe_set_tile_stats", "moe_probe_workgroups", "moe_mfma_probe", "moe_load_probe_bytes", "moe_load_probe",
)
NOALLOC_SCRATCH_BYTES = 4 << 20    # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("T", _i64), ("H", _i64), ("I", _i64),
        ("E", _i32), ("k", _i32), ("compute", _i32), ("io_dtype", _i32),
        ("x", _vp), ("topk_idx", _vp), ("topk_prob", _vp),
        ("w1", ctypes.POINTER(_vp)), ("w2", ctypes.POINTER(_vp)),
        ("out", _vp),
        ("split_sizes", _vp), ("offsets", _vp), ("row_id_map", _vp), ("src_index", _vp), ("prob_perm", _vp),
        ("saved_x_perm", _vp), ("saved_gu", _vp), ("saved_h", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("w1q", _vp), ("w1s", _vp), ("w2q", _vp), ("w2s", _vp),
        ("w1_scale", _vp), ("w2_scale", _vp),
        ("error_flag", _vp), ("h_codes", _vp), ("h_scales", _vp), ("h_f32", _vp),
        ("w1tq_out", _vp), ("w1ts_out", _vp), ("w2tq_out", _vp), ("w2ts_out", _vp),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("T", _i64), ("H", _i64), ("I", _i64),
        ("E", _i32), ("k", _i32), ("compute", _i32), ("io_dtype", _i32), ("dw_dtype", _i32),
        ("dy", _vp),
        ("w1", ctypes.POINTER(_vp)), ("w2", ctypes.POINTER(_vp)),
        ("split_sizes", _vp), ("offsets", _vp), ("row_id_map", _vp), ("src_index", _vp), ("prob_perm", _vp),
        ("saved_x_perm", _vp), ("saved_gu", _vp), ("saved_h", _vp),
        ("dx", _vp), ("dprob", _vp),
        ("dw1", ctypes.POINTER(_vp)), ("dw2", ctypes.POINTER(_vp)),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("w1tq", _vp), ("w1ts", _vp), ("w2tq", _vp), ("w2ts", _vp),
        ("dgu_bf16", _vp), ("dgu_codes", _vp), ("dgu_scales", _vp), ("dgu_t_codes", _vp), ("dgu_t_scales", _vp),
    ]


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m mixture_experts_grouped_permute_amd.build`")
    lib = ctypes.CDLL(p)
    lib.moe_abi_version.restype = ctypes.c_int
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.mxfp8_quantize.restype = ctypes.c_int
    lib.mxfp8_quantize.argtypes = [_vp, ctypes.c_int, _i64, _i64, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp]
    lib.mxfp8_quantize_weights.restype = ctypes.c_int
    lib.mxfp8_quantize_weights.argtypes = [ctypes.POINTER(_vp), ctypes.c_int, _i64, _i64, ctypes.c_int, _vp, _vp,
                                           _vp, _vp]
    lib.fp8_tensor_quantize_workspace.restype = ctypes.c_size_t
    lib.fp8_tensor_quantize_workspace.argtypes = [ctypes.c_int]
    lib.fp8_tensor_quantize.restype = ctypes.c_int
    lib.fp8_tensor_quantize.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, ctypes.c_int, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]
    lib.moe_permute_workspace_size.restype = ctypes.c_size_t
    lib.moe_permute_workspace_size.argtypes = [_i64, ctypes.c_int, ctypes.c_int]
    lib.moe_permute.restype = ctypes.c_int
    lib.moe_permute.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_permute_noalloc.restype = ctypes.c_int
    lib.moe_permute_noalloc.argtypes = [_vp, ctypes.c_int, _i64, _i64, _vp, _vp, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.moe_grouped_mlp_fwd_workspace.restype = ctypes.c_size_t
    lib.moe_grouped_mlp_fwd_workspace.argtypes = [ctypes.POINTER(FwdArgs)]
    lib.moe_grouped_mlp_fwd.restype = ctypes.c_int
    lib.moe_grouped_mlp_fwd.argtypes = [ctypes.POINTER(FwdArgs), _vp]
    lib.moe_grouped_mlp_bwd_workspace.restype = ctypes.c_size_t
    lib.moe_grouped_mlp_bwd_workspace.argtypes = [ctypes.POINTER(BwdArgs)]
    lib.moe_grouped_mlp_bwd.restype = ctypes.c_int
    lib.moe_grouped_mlp_bwd.argtypes = [ctypes.POINTER(BwdArgs), _vp]
    lib.moe_grouped_mlp_fwd_ex.restype = ctypes.c_int
    lib.moe_grouped_mlp_fwd_ex.argtypes = [ctypes.POINTER(FwdArgs), _vp, ctypes.POINTER(_vp)]
    lib.moe_fwd_phase_count.restype = ctypes.c_int
    lib.moe_fwd_phase_name.restype = ctypes.c_char_p
    lib.moe_fwd_phase_name.argtypes = [ctypes.c_int]
    lib.moe_grouped_mlp_bwd_ex.restype = ctypes.c_int
    lib.moe_grouped_mlp_bwd_ex.argtypes = [ctypes.POINTER(BwdArgs), _vp, ctypes.POINTER(_vp)]
    lib.moe_bwd_phase_count.restype = ctypes.c_int
    lib.moe_bwd_phase_name.restype = ctypes.c_char_p
    lib.moe_bwd_phase_name.argtypes = [ctypes.c_int]
    lib.moe_read_device_error.restype = ctypes.c_int
    lib.moe_read_device_error.argtypes = [_vp, _vp]
    lib.moe_probe_workgroups.restype = ctypes.c_int
    lib.moe_mfma_probe.restype = ctypes.c_int
    lib.moe_mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]
    lib.moe_load_probe_bytes.restype = ctypes.c_size_t
    lib.moe_load_probe.restype = ctypes.c_int
    lib.moe_load_probe.argtypes = [ctypes.c_int, ctypes.c_int, _vp, ctypes.c_size_t, _vp, _vp]
    lib.moe_tile_stats_bytes.restype = ctypes.c_size_t
    lib.moe_tile_stats_bytes.argtypes = []
    lib.moe_set_tile_stats.restype = ctypes.c_int
    lib.moe_set_tile_stats.argtypes = [_vp, ctypes.c_size_t]
    lib.moe_grouped_mlp_fwd_loop.restype = ctypes.c_int
    lib.moe_grouped_mlp_fwd_loop.argtypes = [ctypes.POINTER(FwdArgs), ctypes.POINTER(_i32), _vp]
    lib.moe_route_topk.restype = ctypes.c_int
    lib.moe_route_topk.argtypes = [_vp, ctypes.c_int, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]
    lib.moe_route_permute.restype = ctypes.c_int
    lib.moe_route_permute.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_size_t, _vp]
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().moe_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def _check(status: int, what: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, what)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _io(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _compute(c: str) -> int:
    return {"bf16": MOE_BF16, "mxfp8": MOE_MXFP8_E4M3, "fp8": MOE_FP8_E4M3}[c]


def _need(t: Optional[torch.Tensor], dtype: torch.dtype, device: torch.device, what: str) -> None:
    """Raise TypeError unless t is a tensor of `dtype` on `device` (the library reads raw bytes)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise TypeError(f"{what} must be on {device}, got {t.device}")


def _table(ws: Sequence[torch.Tensor] | torch.Tensor, dtype: Optional[torch.dtype] = None,
           device: Optional[torch.device] = None, what: str = "weight"):
    """Host array of the device pointers of ws[e] (a stacked tensor or a list), and the tensors
    behind them: non-contiguous entries are copied, and the copies are returned so that the caller
    keeps them alive until the launch has been enqueued."""
    items = [ws[e] for e in range(ws.shape[0])] if isinstance(ws, torch.Tensor) else list(ws)
    if dtype is not None:
        for w in items:
            _need(w, dtype, device if device is not None else w.device, what)
    items = [w if w.is_contiguous() else w.contiguous() for w in items]
    arr = (_vp * len(items))(*[w.data_ptr() for w in items])
    return arr, items


class _Workspace:
    """A growable scratch buffer per (device, stream), owned by torch (the library never
    allocates).  Calls on one stream run in order, so they can share its buffer; calls on
    different streams get different buffers.  A grown buffer replaces the old one, which stays
    valid for the kernels already enqueued: it was allocated on that same stream, so torch's
    allocator reuses its memory only in that stream's order."""

    def __init__(self):
        self.buf = {}

    def get(self, nbytes: int, device: torch.device) -> torch.Tensor:
        stream = torch.cuda.current_stream(device)
        key = (device.type, device.index, stream.cuda_stream)
        b = self.buf.get(key)
        if b is None or b.numel() < nbytes:
            b = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self.buf[key] = b
        return b


_WS = _Workspace()


# ----------------------------------------------------------------------------- entry points

def mxfp8_quantize(x: torch.Tensor, axis: int = 0, group_offsets: Optional[torch.Tensor] = None):
    """OCP MXFP8 of x [rows, cols] (bf16 or f32).

    axis 0: returns (codes uint8 [rows, cols], scales uint8 [rows, cols/32]).
    axis 1: blocks along rows restarted per segment of group_offsets (int32 device
            [G+1]); returns (codes [cols, rows + 32G], scales [cols, (rows + 32G)/32]),
            token axis contiguous, padded segments as documented in moe.h.
    """
    lib = load()
    rows, cols = x.shape
    dev = x.device
    if axis == 0:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        st = lib.mxfp8_quantize(_ptr(x), _io(x), rows, cols, 0, None, 0, _ptr(q), _ptr(s), _stream(dev))
    else:
        G = group_offsets.numel() - 1
        rp = (rows + 31) // 32 * 32 + 32 * G
        q = torch.empty((cols, rp), dtype=torch.uint8, device=dev)      # every byte is written
        s = torch.empty((cols, rp // 32), dtype=torch.uint8, device=dev)
        st = lib.mxfp8_quantize(_ptr(x), _io(x), rows, cols, 1, _ptr(group_offsets), G, _ptr(q), _ptr(s),
                                _stream(dev))
    _check(st, "mxfp8_quantize")
    return q, s


def fp8_tensor_quantize(x: torch.Tensor, group_offsets: Optional[torch.Tensor] = None):
    """Per-tensor-scaled E4M3 of x [rows, cols] (bf16 or f32): one fp32 scale per row segment of
    group_offsets (int32 device [G+1]), or one for all of x.  Returns (codes uint8 [rows, cols],
    scales float32 [G]); a code stands for decode(code) / scale."""
    lib = load()
    rows, cols = x.shape
    dev = x.device
    G = 1 if group_offsets is None else group_offsets.numel() - 1
    q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    s = torch.empty(G, dtype=torch.float32, device=dev)
    need = lib.fp8_tensor_quantize_workspace(G)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.fp8_tensor_quantize(_ptr(x), _io(x), rows, cols, _ptr(group_offsets), G, _ptr(q), _ptr(s),
                                 _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "fp8_tensor_quantize")
    return q, s


def _check_routing(topk_idx: torch.Tensor, topk_prob: Optional[torch.Tensor], device: torch.device) -> None:
    _need(topk_idx, torch.int32, device, "topk_idx")
    _need(topk_prob, torch.float32, device, "topk_prob")


def _perm_outputs(T: int, k: int, E: int, dev: torch.device, prob: bool = True) -> dict:
    R = T * k
    return {
        "split_sizes": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "row_id_map": torch.empty(R, dtype=torch.int32, device=dev),
        "src_index": torch.empty(R, dtype=torch.int32, device=dev),
        "prob_perm": torch.empty(R, dtype=torch.float32, device=dev) if prob else None,
    }


def moe_permute(x: Optional[torch.Tensor], topk_idx: torch.Tensor, topk_prob: Optional[torch.Tensor], E: int,
                perm_dtype: str = "bf16"):
    """Histogram / prefix sum / stable scatter.  Returns a dict of device tensors; its
    "workspace" entry (this call's own) holds the bad-expert-id flag in its first 4 bytes."""
    lib = load()
    T, k = topk_idx.shape
    dev = topk_idx.device
    _check_routing(topk_idx, topk_prob, dev)
    R = T * k
    out = _perm_outputs(T, k, E, dev, topk_prob is not None)
    out["x_perm"], out["x_perm_scales"] = None, None
    H = 0
    pd = _compute(perm_dtype)
    if x is not None:
        if x.device != dev:
            raise TypeError(f"x must be on {dev}")
        H = x.shape[1]
        if pd == MOE_BF16:
            out["x_perm"] = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        else:
            out["x_perm"] = torch.empty((R, H), dtype=torch.uint8, device=dev)
            out["x_perm_scales"] = torch.empty((R, H // 32), dtype=torch.uint8, device=dev)
    # the index workspace is small: one per call, so the flag it holds stays this call's
    need = lib.moe_permute_workspace_size(T, k, E)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.moe_permute(_ptr(x), _io(x) if x is not None else MOE_BF16, T, H, _ptr(topk_idx), _ptr(topk_prob),
                         k, E, pd, _ptr(out["x_perm"]), _ptr(out["x_perm_scales"]), _ptr(out["split_sizes"]),
                         _ptr(out["offsets"]), _ptr(out["row_id_map"]), _ptr(out["src_index"]),
                         _ptr(out["prob_perm"]), ws.data_ptr(), ws.numel(), _stream(dev))
    _check(st, "moe_permute")
    out["workspace"] = ws
    return out


def moe_permute_noalloc(x: Optional[torch.Tensor], topk_idx: torch.Tensor, topk_prob: Optional[torch.Tensor],
                        E: int, perm_dtype: str = "bf16", out: Optional[dict] = None):
    """moe_permute through the entry point that allocates nothing (its index scratch is the
    library's fixed device array).  `out`: optional dict of preallocated output tensors with
    moe_permute's keys plus "error_flag" (int32 [1]); missing ones are allocated here, by torch,
    before the call.  Returns the dict."""
    lib = load()
    T, k = topk_idx.shape
    dev = topk_idx.device
    _check_routing(topk_idx, topk_prob, dev)
    R = T * k
    res = dict(out) if out is not None else {}
    for key, t in _perm_outputs(T, k, E, dev, topk_prob is not None).items():
        res.setdefault(key, t)
    res.setdefault("error_flag", torch.zeros(1, dtype=torch.int32, device=dev))
    H = 0
    pd = _compute(perm_dtype)
    if x is not None:
        H = x.shape[1]
        if pd == MOE_BF16:
            res.setdefault("x_perm", torch.empty((R, H), dtype=torch.bfloat16, device=dev))
        else:
            res.setdefault("x_perm", torch.empty((R, H), dtype=torch.uint8, device=dev))
            res.setdefault("x_perm_scales", torch.empty((R, H // 32), dtype=torch.uint8, device=dev))
    res.setdefault("x_perm", None)
    res.setdefault("x_perm_scales", None)
    st = lib.moe_permute_noalloc(_ptr(x), _io(x) if x is not None else MOE_BF16, T, H, _ptr(topk_idx),
                                 _ptr(topk_prob), k, E, pd, _ptr(res["x_perm"]), _ptr(res["x_perm_scales"]),
                                 _ptr(res["split_sizes"]), _ptr(res["offsets"]), _ptr(res["row_id_map"]),
                                 _ptr(res["src_index"]), _ptr(res["prob_perm"]), _ptr(res["error_flag"]),
                                 _stream(dev))
    _check(st, "moe_permute_noalloc")
    return res


def moe_route_topk(logits: torch.Tensor, k: int):
    """Top-k router: returns (topk_idx int32 [T,k], topk_prob float32 [T,k])."""
    lib = load()
    T, E = logits.shape
    dev = logits.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    prob = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib.moe_route_topk(_ptr(logits), _io(logits), T, E, k, _ptr(idx), _ptr(prob), _stream(dev)),
           "moe_route_topk")
    return idx, prob


def moe_route_permute(logits: torch.Tensor, x: Optional[torch.Tensor], k: int, perm_dtype: str = "bf16"):
    """Router fused with the permutation.  Returns moe_permute's dict plus topk_idx / topk_prob."""
    lib = load()
    T, E = logits.shape
    dev = logits.device
    R = T * k
    out = {
        "topk_idx": torch.empty((T, k), dtype=torch.int32, device=dev),
        "topk_prob": torch.empty((T, k), dtype=torch.float32, device=dev),
        **_perm_outputs(T, k, E, dev),
        "x_perm": None, "x_perm_scales": None,
    }
    H = 0
    pd = _compute(perm_dtype)
    if x is not None:
        if x.device != dev:
            raise TypeError(f"x must be on {dev}")
        H = x.shape[1]
        if pd == MOE_BF16:
            out["x_perm"] = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        else:
            out["x_perm"] = torch.empty((R, H), dtype=torch.uint8, device=dev)
            out["x_perm_scales"] = torch.empty((R, H // 32), dtype=torch.uint8, device=dev)
    need = lib.moe_permute_workspace_size(T, k, E)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.moe_route_permute(_ptr(logits), _io(logits), _ptr(x), _io(x) if x is not None else MOE_BF16, T, H, E, k,
                               pd, _ptr(out["topk_idx"]), _ptr(out["topk_prob"]), _ptr(out["x_perm"]),
                               _ptr(out["x_perm_scales"]), _ptr(out["split_sizes"]), _ptr(out["offsets"]),
                               _ptr(out["row_id_map"]), _ptr(out["src_index"]), _ptr(out["prob_perm"]),
                               ws.data_ptr(), ws.numel(), _stream(dev))
    _check(st, "moe_route_permute")
    out["workspace"] = ws
    return out


def _fwd_args(x, topk_idx, topk_prob, w1, w2, compute, out, perm, saved):
    """Argument struct of a forward call (no launch) and the tensors it points into."""
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    _io(x)
    _check_routing(topk_idx, topk_prob, dev)
    w1t, w1k = _table(w1, torch.bfloat16, dev, "w1")
    w2t, w2k = _table(w2, torch.bfloat16, dev, "w2")
    E = len(w1k)
    if len(w2k) != E:
        raise ValueError("w1 and w2 must hold the same number of experts")
    I = w2k[0].shape[1]
    a = FwdArgs()
    a.T, a.H, a.I, a.E, a.k = T, H, I, E, k
    a.compute = _compute(compute)
    a.io_dtype = _io(x)
    a.x, a.topk_idx, a.topk_prob = _ptr(x), _ptr(topk_idx), _ptr(topk_prob)
    a.w1, a.w2 = w1t, w2t
    a.out = _ptr(out)
    a.split_sizes, a.offsets = _ptr(perm["split_sizes"]), _ptr(perm["offsets"])
    a.row_id_map, a.src_index, a.prob_perm = _ptr(perm["row_id_map"]), _ptr(perm["src_index"]), _ptr(perm["prob_perm"])
    if saved is not None:
        a.saved_x_perm, a.saved_gu, a.saved_h = _ptr(saved["x_perm"]), _ptr(saved["gu"]), _ptr(saved["h"])
    return a, (w1t, w2t, w1k, w2k), E, I


def mxfp8_quantize_weights(w, axis: int = 0, skip: Optional[torch.Tensor] = None):
    """OCP MXFP8 of E bf16 matrices [rows, cols] (a stacked tensor or a list) in one launch.
    axis 0: (codes [E, rows, cols], scales [E, rows, cols/32]);
    axis 1: transposed, (codes [E, cols, rows], scales [E, cols, rows/32]).
    skip: optional int32 device [E]; matrices with skip[e] == 0 are left as zeros."""
    lib = load()
    tab, items = _table(w, torch.bfloat16, None, "w")
    E = len(items)
    rows, cols = items[0].shape
    dev = items[0].device
    for t in items:
        if t.shape != (rows, cols) or t.device != dev:
            raise ValueError("every matrix must have the same shape and device")
    _need(skip, torch.int32, dev, "skip")
    shape = (E, rows, cols) if axis == 0 else (E, cols, rows)
    make = torch.zeros if skip is not None else torch.empty
    q = make(shape, dtype=torch.uint8, device=dev)
    s = make((shape[0], shape[1], shape[2] // 32), dtype=torch.uint8, device=dev)
    _check(lib.mxfp8_quantize_weights(tab, E, rows, cols, axis, _ptr(skip), _ptr(q), _ptr(s), _stream(dev)),
           "mxfp8_quantize_weights")
    return q, s


def quantize_weights(w1, w2, compute: str = "mxfp8", transposed: bool = False):
    """Quantized weights for reuse across calls.
    "mxfp8": (w1q [E,2I,H], w1s [E,2I,H/32], w2q [E,H,I], w2s [E,H,I/32]), every expert quantized
    row-wise by the kernel the forward runs per call (mxfp8_quantize_weights, axis 0).
    "mxfp8", transposed=True: the backward's dgrad operands, (w1tq [E,H,2I], w1ts [E,H,2I/32],
    w2tq [E,I,H], w2ts [E,I,H/32]) (axis 1).
    "fp8": (w1q [E,2I,H], w1_scale [E], w2q [E,H,I], w2_scale [E]), each expert's matrix one
    tensor of fp8_tensor_quantize."""
    if compute == "fp8":
        if transposed:
            raise ValueError("the per-tensor FP8 variant is forward only")
        e1 = [w1[e] for e in range(len(w1))]
        e2 = [w2[e] for e in range(len(w2))]
        q1 = [fp8_tensor_quantize(w) for w in e1]
        q2 = [fp8_tensor_quantize(w) for w in e2]
        return (torch.stack([q for q, _ in q1]), torch.cat([s for _, s in q1]),
                torch.stack([q for q, _ in q2]), torch.cat([s for _, s in q2]))
    if compute != "mxfp8":
        raise ValueError(f"no cached weights for compute {compute!r}")
    axis = 1 if transposed else 0
    w1q, w1s = mxfp8_quantize_weights(w1, axis)
    w2q, w2s = mxfp8_quantize_weights(w2, axis)
    return w1q, w1s, w2q, w2s


def moe_grouped_mlp_fwd(x: torch.Tensor, topk_idx: torch.Tensor, topk_prob: torch.Tensor, w1, w2,
                        compute: str = "bf16", save_for_backward: bool = False, workspace: Optional[torch.Tensor] = None,
                        w_quant=None, debug_h: bool = False, quantize_for_backward: Optional[bool] = None):
    """Grouped expert MLP forward.  w1: [E,2I,H] tensor or E tensors [2I,H] (bf16);
    w2: [E,H,I] or E tensors [H,I].  compute: "bf16", "mxfp8" or "fp8" (per-tensor scales,
    forward only).  w_quant: optional quantize_weights(w1, w2, compute) output ("mxfp8" or
    "fp8"): the per-call weight quantization is skipped.
    quantize_for_backward (MXFP8 with save_for_backward and per-call weight quantization; the
    default there): the same read of the bf16 weights also quantizes them along the backward's K,
    into ctx["w_quant_t"], which moe_grouped_mlp_bwd then uses.
    debug_h: also return, in ctx["debug"], h in fp32 as FC1's epilogue computed it ("h_f32",
    [R, I], permuted rows) and, under MXFP8, the E4M3 codes and E8M0 scales its fused quantizer
    wrote ("h_codes" [R, I], "h_scales" [R, I/32]).
    Returns (out, ctx) where ctx holds the permutation, the bad-expert-id flag ("error_flag")
    and, with save_for_backward, the bf16 activations."""
    lib = load()
    dev = x.device
    T, H = x.shape
    k = topk_idx.shape[1]
    R = T * k
    E = w1.shape[0] if isinstance(w1, torch.Tensor) else len(w1)
    I = (w2.shape[2] if isinstance(w2, torch.Tensor) else w2[0].shape[1])
    perm = _perm_outputs(T, k, E, dev)
    saved = None
    if save_for_backward:
        saved = {
            "x_perm": torch.empty((R, H), dtype=torch.bfloat16, device=dev),
            "gu": torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev),
            "h": torch.empty((R, I), dtype=torch.bfloat16, device=dev),
        }
    out = torch.empty((T, H), dtype=x.dtype, device=dev)
    a, keep, _, _ = _fwd_args(x, topk_idx, topk_prob, w1, w2, compute, out, perm, saved)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    a.error_flag = flag.data_ptr()
    debug = None
    if debug_h:
        debug = {"h_f32": torch.empty((R, I), dtype=torch.float32, device=dev)}
        a.h_f32 = debug["h_f32"].data_ptr()
        if compute == "mxfp8":
            debug["h_codes"] = torch.empty((R, I), dtype=torch.uint8, device=dev)
            debug["h_scales"] = torch.empty((R, I // 32), dtype=torch.uint8, device=dev)
            a.h_codes, a.h_scales = debug["h_codes"].data_ptr(), debug["h_scales"].data_ptr()
    wqt = None
    if quantize_for_backward is None:
        quantize_for_backward = save_for_backward and compute == "mxfp8" and w_quant is None
    if quantize_for_backward:
        if not (save_for_backward and compute == "mxfp8" and w_quant is None):
            raise ValueError("quantize_for_backward needs save_for_backward, mxfp8 and per-call weights")
        u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device=dev)
        Hh = x.shape[1]
        wqt = (u8(E, Hh, 2 * I), u8(E, Hh, 2 * I // 32), u8(E, I, Hh), u8(E, I, Hh // 32))
        a.w1tq_out, a.w1ts_out, a.w2tq_out, a.w2ts_out = (t.data_ptr() for t in wqt)
    if w_quant is not None:
        for t in w_quant:
            if t.device != dev:
                raise TypeError(f"cached weights must be on {dev}")
        if compute == "fp8":
            a.w1q, a.w1_scale, a.w2q, a.w2_scale = (_ptr(t) for t in w_quant)
        else:
            a.w1q, a.w1s, a.w2q, a.w2s = (_ptr(t) for t in w_quant)
        keep = (keep, w_quant)
    need = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
    if need == 0:
        # the size query validates the arguments: surface the status of the call itself
        _check(lib.moe_grouped_mlp_fwd(ctypes.byref(a), _stream(dev)), "moe_grouped_mlp_fwd")
    ws = workspace if workspace is not None else _WS.get(need, dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    _check(lib.moe_grouped_mlp_fwd(ctypes.byref(a), _stream(dev)), "moe_grouped_mlp_fwd")
    ctx = {"perm": perm, "saved": saved, "compute": compute, "E": E, "I": I, "error_flag": flag,
           "workspace": ws, "_keep": keep, "w_quant_t": wqt}
    if debug is not None:
        ctx["debug"] = debug
    return out, ctx


def moe_grouped_mlp_fwd_loop(x: torch.Tensor, topk_idx: torch.Tensor, topk_prob: torch.Tensor, w1, w2,
                             split_sizes_host: Sequence[int], compute: str = "bf16"):
    """The same forward as a per-expert loop of launches (the baseline grouping replaces).
    split_sizes_host: the per-expert token counts of topk_idx, on the host."""
    lib = load()
    dev = x.device
    T, H = x.shape
    k = topk_idx.shape[1]
    E = w1.shape[0] if isinstance(w1, torch.Tensor) else len(w1)
    perm = _perm_outputs(T, k, E, dev)
    out = torch.empty((T, H), dtype=x.dtype, device=dev)
    a, keep, _, _ = _fwd_args(x, topk_idx, topk_prob, w1, w2, compute, out, perm, None)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    a.error_flag = flag.data_ptr()
    need = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
    if need == 0:
        _check(lib.moe_grouped_mlp_fwd(ctypes.byref(a), _stream(dev)), "moe_grouped_mlp_fwd_loop")
    ws = _WS.get(need, dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    counts = (_i32 * E)(*[int(c) for c in split_sizes_host])
    _check(lib.moe_grouped_mlp_fwd_loop(ctypes.byref(a), counts, _stream(dev)), "moe_grouped_mlp_fwd_loop")
    return out, {"perm": perm, "error_flag": flag, "workspace": ws, "_keep": keep}


def _bwd_args(dy: torch.Tensor, ctx: dict, w1, w2, dw_dtype=torch.float32, w_quant_t=None):
    """Output tensors and the argument struct of a backward call (no launch)."""
    dev = dy.device
    T, H = dy.shape
    perm, saved = ctx["perm"], ctx["saved"]
    if saved is None:
        raise ValueError("forward was run without save_for_backward")
    _io(dy)
    E, I = ctx["E"], ctx["I"]
    k = perm["row_id_map"].numel() // T
    dx = torch.empty((T, H), dtype=dy.dtype, device=dev)
    dprob = torch.empty((T, k), dtype=torch.float32, device=dev)
    dw1 = torch.empty((E, 2 * I, H), dtype=dw_dtype, device=dev)
    dw2 = torch.empty((E, H, I), dtype=dw_dtype, device=dev)
    w1t, w1k = _table(w1, torch.bfloat16, dev, "w1")
    w2t, w2k = _table(w2, torch.bfloat16, dev, "w2")
    dw1t, _ = _table(dw1)
    dw2t, _ = _table(dw2)
    a = BwdArgs()
    a.T, a.H, a.I, a.E, a.k = T, H, I, E, k
    a.compute = _compute(ctx["compute"])
    a.io_dtype = _io(dy)
    a.dw_dtype = _io(dw1)
    a.dy = _ptr(dy)
    a.w1, a.w2 = w1t, w2t
    a.split_sizes, a.offsets = _ptr(perm["split_sizes"]), _ptr(perm["offsets"])
    a.row_id_map, a.src_index, a.prob_perm = _ptr(perm["row_id_map"]), _ptr(perm["src_index"]), _ptr(perm["prob_perm"])
    a.saved_x_perm, a.saved_gu, a.saved_h = _ptr(saved["x_perm"]), _ptr(saved["gu"]), _ptr(saved["h"])
    a.dx, a.dprob = _ptr(dx), _ptr(dprob)
    a.dw1, a.dw2 = dw1t, dw2t
    if w_quant_t is None:
        w_quant_t = ctx.get("w_quant_t")   # quantized by the forward, if it was asked to
    if w_quant_t is not None:
        for t in w_quant_t:
            _need(t, torch.uint8, dev, "cached transposed weights")
        a.w1tq, a.w1ts, a.w2tq, a.w2ts = (_ptr(t) for t in w_quant_t)
    return a, (dx, dprob, dw1, dw2), (w1t, w2t, dw1t, dw2t, w1k, w2k, w_quant_t)


def moe_grouped_mlp_bwd(dy: torch.Tensor, ctx: dict, w1, w2, dw_dtype=torch.float32,
                        workspace: Optional[torch.Tensor] = None, w_quant_t=None, debug: Optional[dict] = None):
    """Backward of moe_grouped_mlp_fwd (needs save_for_backward=True).
    w_quant_t: optional quantize_weights(w1, w2, "mxfp8", transposed=True) output (MXFP8): the
    per-call quantization of the transposed weights is skipped.
    debug: optional dict (MXFP8): filled with the FC2 dgrad epilogue's dgu in bf16 ("dgu_bf16"
    [R, 2I]) and its two quantizations ("dgu_codes", "dgu_scales" row-wise; "dgu_t_codes",
    "dgu_t_scales" along tokens, [2I, rows_pad] with rows_pad = ceil(R/128)*128 + 128 E rounded up to
    a multiple of 512).
    Returns (dx [T,H], dprob [T,k] f32, dw1 [E,2I,H], dw2 [E,H,I])."""
    lib = load()
    dev = dy.device
    a, outs, keep = _bwd_args(dy, ctx, w1, w2, dw_dtype, w_quant_t)
    dx, dprob, dw1, dw2 = outs
    if debug is not None:
        R, I2, E = int(a.T) * int(a.k), 2 * int(a.I), int(a.E)
        rp = ((R + 127) // 128 * 128 + 128 * E + 511) // 512 * 512
        u8 = lambda *shape: torch.zeros(shape, dtype=torch.uint8, device=dev)
        debug.update(dgu_bf16=torch.zeros((R, I2), dtype=torch.bfloat16, device=dev), dgu_codes=u8(R, I2),
                     dgu_scales=u8(R, I2 // 32), dgu_t_codes=u8(I2, rp), dgu_t_scales=u8(I2, rp // 32))
        for name in ("dgu_bf16", "dgu_codes", "dgu_scales", "dgu_t_codes", "dgu_t_scales"):
            setattr(a, name, debug[name].data_ptr())
    need = lib.moe_grouped_mlp_bwd_workspace(ctypes.byref(a))
    if need == 0:
        _check(lib.moe_grouped_mlp_bwd(ctypes.byref(a), _stream(dev)), "moe_grouped_mlp_bwd")
    ws = workspace if workspace is not None else _WS.get(need, dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    _check(lib.moe_grouped_mlp_bwd(ctypes.byref(a), _stream(dev)), "moe_grouped_mlp_bwd")
    del keep
    return dx, dprob, dw1, dw2


TILE_STAT_SLOTS = ("fc1", "fc2", "dgrad_fc2", "wgrad_fc2", "dgrad_fc1", "wgrad_fc1")


def set_tile_stats(buf: Optional[torch.Tensor]) -> None:
    """Diagnostic: record per-wave GEMM cycle counts into `buf` (an int32 device tensor of at least
    moe_tile_stats_bytes() bytes) on later calls, or stop (None).  Process-wide; see moe.h."""
    lib = load()
    if buf is None:
        _check(lib.moe_set_tile_stats(None, 0), "moe_set_tile_stats")
        return
    if buf.dtype != torch.int32 or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("tile stats buffer must be a contiguous int32 device tensor")
    _check(lib.moe_set_tile_stats(_ptr(buf), buf.numel() * 4), "moe_set_tile_stats")


def tile_stats_new(device) -> torch.Tensor:
    """A zeroed buffer for set_tile_stats."""
    return torch.zeros(load().moe_tile_stats_bytes() // 4, dtype=torch.int32, device=device)


def tile_stats_summary(buf: torch.Tensor) -> dict:
    """Per GEMM slot recorded in `buf`: work items per wave (min, max), mean main-loop and epilogue
    cycles per item, and the slowest wave's total cycles."""
    import numpy as np
    w = buf.view(len(TILE_STAT_SLOTS), -1, 4).cpu().numpy().astype(np.uint32).astype(np.float64)
    out = {}
    for k, name in enumerate(TILE_STAT_SLOTS):
        v = w[k]
        if not (v[:, 3] == 0x7153).all():
            continue
        items = v[:, 2]
        n = max(items.sum(), 1.0)
        out[name] = {"items_per_wave": [int(items.min()), int(items.max())],
                     "main_cycles_per_item": round(v[:, 0].sum() / n),
                     "epilogue_cycles_per_item": round(v[:, 1].sum() / n),
                     "epilogue_frac": round(v[:, 1].sum() / max(v[:, 0].sum() + v[:, 1].sum(), 1.0), 4),
                     "max_wave_cycles": int((v[:, 0] + v[:, 1]).max()),
                     "mean_wave_cycles": round((v[:, 0] + v[:, 1]).mean())}
    return out


MFMA_PROBE_KINDS = ("mfma_scale_32x32x64_e4m3", "mfma_scale_32x32x64_e4m3_const_scales", "mfma_32x32x16_bf16",
                    "mfma_32x32x16_bf16_random_4x4_fragments", "mfma_scale_32x32x64_e4m3_random_4x4_fragments")


def mfma_probe(kind: int, iters: int = 2000, device="cuda:0", reps: int = 3) -> dict:
    """Diagnostic: back-to-back MFMA issue cost on every SIMD (moe_mfma_probe).  Returns the mean
    and max shader-clock cycles per MFMA over the 1024 waves, the launch time (median of `reps`
    event-timed launches after one warm-up), the clock that implies, and the dense rate."""
    lib = load()
    dev = torch.device(device)
    G = lib.moe_probe_workgroups()
    sink = torch.empty(G * 256, dtype=torch.float32, device=dev)
    cyc = torch.zeros(G * 4, dtype=torch.int64, device=dev)
    ms = []
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _check(lib.moe_mfma_probe(kind, iters, _ptr(sink), _ptr(cyc), _stream(dev)), "moe_mfma_probe")
        e1.record()
        torch.cuda.synchronize(dev)
        if r:
            ms.append(e0.elapsed_time(e1))
    ms.sort()
    t = ms[len(ms) // 2]
    c = cyc.cpu().double()
    per = c / (16.0 * iters)
    flop = (32 * 32 * 16 * 2) if kind in (2, 3) else (32 * 32 * 64 * 2)
    return {"kind": MFMA_PROBE_KINDS[kind], "iters": iters, "waves": G * 4,
            "cycles_per_mfma_mean": round(float(per.mean()), 2), "cycles_per_mfma_max": round(float(per.max()), 2),
            "launch_ms": round(t, 4), "clock_ghz": round(float(c.mean()) / (t * 1e6), 3),
            "tflops": round(flop * 16.0 * iters * G * 4 / (t * 1e-3) / 1e12, 1)}


LOAD_PROBE_PATTERNS = ("own_chunks_l2_resident", "own_chunks_streamed", "8_sharers_lockstep_streamed",
                       "8_sharers_gemm_rows_streamed")


def load_probe(pattern: int, stages: int = 512, device="cuda:0", reps: int = 3, buf: Optional[torch.Tensor] = None) -> dict:
    """Diagnostic: the LDS fill rate of the GEMMs' direct-to-LDS loads (moe_load_probe).  Returns the
    launch time (median of `reps` event-timed launches after one warm-up), the bytes per cycle and
    per CU (mean over the 256 workgroups' shader-clock cycles), and the aggregate rate into LDS."""
    lib = load()
    dev = torch.device(device)
    need = lib.moe_load_probe_bytes()
    if buf is None:
        buf = torch.zeros(need, dtype=torch.uint8, device=dev)
    if buf.numel() < need or not buf.is_cuda:
        raise TypeError(f"load probe buffer must be a device tensor of at least {need} bytes")
    cyc = torch.zeros(256, dtype=torch.int64, device=dev)
    ms = []
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _check(lib.moe_load_probe(pattern, stages, _ptr(buf), buf.numel(), _ptr(cyc), _stream(dev)), "moe_load_probe")
        e1.record()
        torch.cuda.synchronize(dev)
        if r:
            ms.append(e0.elapsed_time(e1))
    ms.sort()
    t = ms[len(ms) // 2]
    c = float(cyc.cpu().double().mean())
    return {"pattern": LOAD_PROBE_PATTERNS[pattern], "stages": stages, "launch_ms": round(t, 4),
            "bytes_per_cycle_per_cu": round(65536.0 * stages / c, 1), "cycles_per_64KB_stage": round(c / stages),
            "TBs_into_lds": round(256 * 65536.0 * stages / (t * 1e-3) / 1e12, 2)}


def moe_read_device_error(flag: torch.Tensor) -> int:
    """The bad-expert-id flag of a call: ctx["error_flag"] of a forward, or the "workspace" of a
    moe_permute / moe_route_permute result (synchronizes the current stream)."""
    return load().moe_read_device_error(flag.data_ptr(), _stream(flag.device))
