#!/usr/bin/env python3
"""Benchmark of the grouped expert MLP forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-mxfp8] [--no-cpu-baseline]

A step is one moe_grouped_mlp_fwd call over the Mixtral-8x7B-shaped layer
(T=4096 tokens, H=4096, I=14336, 8 experts, top-2, bf16 with fp32
accumulation): permutation, FC1 grouped GEMM with ScaledSwiGLU*prob, FC2
grouped GEMM and combine.  Inputs are synthetic (seeded), resident in HBM
before the timed region.  The same line also carries the MXFP8 layer
(T=8192, Zipf(1.2) routing with one empty expert, weights quantized per call)
and the fp64 CPU oracle timed on a bounded sample on the host cores.

Prints one JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE grouped-MLP fwd tokens/s + TFLOP/s (bf16, MXFP8), Mixtral 8x7B layer"
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "fp8": 5000.0}      # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _hip():
    lib = ctypes.CDLL("libamdhip64.so.7")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def _src_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mixture_experts_grouped_permute_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel source changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get(kernel_key)
    if not ent or ent.get("src_hash") != _src_hash(ent.get("sources", ["gemm.hip"])):
        return None
    return ent.get("bytes_per_launch")


def _stats(xs):
    """median, p10 and p90 of a list of floats (nearest-rank)."""
    ys = sorted(xs)
    pick = lambda q: ys[min(len(ys) - 1, max(0, int(round(q * (len(ys) - 1)))))]
    return {"median": round(pick(0.5), 4), "p10": round(pick(0.1), 4), "p90": round(pick(0.9), 4)}


def _time_ex(lib, hip, call_ex, nph, steps, warmup, flush=None):
    """Run call_ex(events) warmup + steps times.  Returns (host ms/step, per-step list of phase ms,
    per-step GPU ms from the first to the last event).  flush(): run before every timed step (outside
    its events, on the same stream) to evict the caches; the host time then includes it."""
    import torch
    ev = []
    for _ in range(steps * (nph + 1)):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        ev.append(e.value)
    arrays = [(ctypes.c_void_p * (nph + 1))(*ev[s * (nph + 1):(s + 1) * (nph + 1)]) for s in range(steps)]
    for _ in range(warmup):
        call_ex(None)
    torch.cuda.synchronize()
    _log(f"timing {steps} steps" + (" (cold caches)" if flush else ""))
    t0 = time.perf_counter()
    for s in range(steps):
        if flush is not None:
            flush()
        call_ex(arrays[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    f = ctypes.c_float()
    per_step, step_ms = [], []
    for s in range(steps):
        row = []
        for i in range(nph):
            hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(arrays[s][i]), ctypes.c_void_p(arrays[s][i + 1]))
            row.append(f.value)
        per_step.append(row)
        hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(arrays[s][0]), ctypes.c_void_p(arrays[s][nph]))
        step_ms.append(f.value)
    for e in ev:
        hip.hipEventDestroy(ctypes.c_void_p(e))
    return (t1 - t0) * 1e3 / steps, per_step, step_ms


def _flusher():
    """A 1 GiB write between timed steps: more than the 256 MB Infinity Cache and the L2s."""
    import torch
    buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    return lambda: buf.fill_(1.0)


TILE_STATS = True   # bench.py --no-tile-stats turns it off


def run_gpu(cfg, steps, warmup, backward=False, cached=False, cold_steps=0, per_call_wt=False):
    import torch
    import mixture_experts_grouped_permute_amd as m
    from mixture_experts_grouped_permute_amd import _lib as L
    from moe_inputs import make_inputs

    lib = m.load()
    hip = _hip()
    _log(f"generating inputs for {cfg.name}")
    inp = make_inputs(cfg, with_dy=backward)
    d = inp.to("cuda:0")
    _log("inputs resident on the GPU; warming up")
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    R = T * k
    dev = d.x.device
    stream = torch.cuda.current_stream(dev).cuda_stream
    if not backward:
        perm = {
            "split_sizes": torch.empty(E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "row_id_map": torch.empty(R, dtype=torch.int32, device=dev),
            "src_index": torch.empty(R, dtype=torch.int32, device=dev),
            "prob_perm": torch.empty(R, dtype=torch.float32, device=dev),
        }
        out = torch.empty((T, H), dtype=d.x.dtype, device=dev)
        a, keep, _, _ = L._fwd_args(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, cfg.precision, out, perm, None)
        if cached:   # weights quantized once, outside the timed region
            wq = m.quantize_weights(d.w1, d.w2, cfg.precision)
            if cfg.precision == "fp8":
                a.w1q, a.w1_scale, a.w2q, a.w2_scale = (t.data_ptr() for t in wq)
            else:
                a.w1q, a.w1s, a.w2q, a.w2s = (t.data_ptr() for t in wq)
            keep = (keep, wq)
        need = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a))
        if need == 0:
            raise RuntimeError("argument validation failed")
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        nph = lib.moe_fwd_phase_count()
        names = [lib.moe_fwd_phase_name(i).decode() for i in range(nph)]

        def call(evs):
            L._check(lib.moe_grouped_mlp_fwd_ex(ctypes.byref(a), stream, evs), "fwd")
    else:
        # MXFP8 training: by default the forward quantizes the weights along the backward's K too
        # (one read of the bf16 masters for both); per_call_wt: the backward quantizes them itself
        qfb = (not per_call_wt) if cfg.precision == "mxfp8" else None
        _, ctx = m.moe_grouped_mlp_fwd(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, cfg.precision,
                                       save_for_backward=True, quantize_for_backward=qfb)
        perm = ctx["perm"]
        # the forward as a training step runs it (saving for the backward), timed the same way
        fout = torch.empty((T, H), dtype=d.x.dtype, device=dev)
        fa, fkeep, _, _ = L._fwd_args(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, cfg.precision, fout, perm,
                                      ctx["saved"])
        if ctx.get("w_quant_t") is not None:
            fa.w1tq_out, fa.w1ts_out, fa.w2tq_out, fa.w2ts_out = (t.data_ptr() for t in ctx["w_quant_t"])
        fneed = lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(fa))
        if fneed == 0:
            raise RuntimeError("argument validation failed")
        fws = torch.empty(fneed, dtype=torch.uint8, device=dev)
        fa.workspace, fa.workspace_bytes = fws.data_ptr(), fws.numel()
        fnph = lib.moe_fwd_phase_count()
        fnames = [lib.moe_fwd_phase_name(i).decode() for i in range(fnph)]

        def fcall(evs):
            L._check(lib.moe_grouped_mlp_fwd_ex(ctypes.byref(fa), stream, evs), "fwd")
        _log("timing the forward that saves for the backward")
        fms, fper, _ = _time_ex(lib, hip, fcall, fnph, steps, warmup)
        fwd_save = {"ms_per_step": fms,
                    "phase_ms": {n: sum(r[i] for r in fper) / len(fper) for i, n in enumerate(fnames)}}
        del fws, fkeep
        a, outs, keep = L._bwd_args(d.dy, ctx, d.w1, d.w2, torch.float32)
        need = lib.moe_grouped_mlp_bwd_workspace(ctypes.byref(a))
        if need == 0:
            raise RuntimeError("argument validation failed")
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        nph = lib.moe_bwd_phase_count()
        names = [lib.moe_bwd_phase_name(i).decode() for i in range(nph)]

        def call(evs):
            L._check(lib.moe_grouped_mlp_bwd_ex(ctypes.byref(a), stream, evs), "bwd")
    ms, per_step, step_ms = _time_ex(lib, hip, call, nph, steps, warmup)
    mean = [sum(r[i] for r in per_step) / len(per_step) for i in range(nph)]
    res = {"ms_per_step": ms, "phase_ms": dict(zip(names, mean)),
           "stats": {"step_gpu_ms": _stats(step_ms),
                     "phase_ms": {n: _stats([r[i] for r in per_step]) for i, n in enumerate(names)}}}
    if cold_steps:
        fl = _flusher()
        _, cold_ph, cold_step = _time_ex(lib, hip, call, nph, cold_steps, 1, flush=fl)
        del fl
        res["cold"] = {"step_gpu_ms": _stats(cold_step),
                       "phase_ms": {n: _stats([r[i] for r in cold_ph]) for i, n in enumerate(names)}}
    # the grouped GEMMs' per-wave cycle split (main loops vs epilogues, shader clock), from one more
    # call outside the timed region with the library's diagnostic counters on
    res["tile_cycles"] = None
    if TILE_STATS:
        tbuf = m.tile_stats_new(dev)
        m.set_tile_stats(tbuf)
        try:
            if backward:
                fcall(None)
            call(None)
            torch.cuda.synchronize()
        finally:
            m.set_tile_stats(None)
        res["tile_cycles"] = m.tile_stats_summary(tbuf)
    res["split_sizes"] = perm["split_sizes"].cpu().tolist()
    res["inputs"] = inp
    if backward:
        res["fwd_save"] = fwd_save
    del keep
    return res


def gemm_roofline(cfg, phase_ms, phase, flops, kernel):
    t = phase_ms[phase] * 1e-3
    ach = flops / t / 1e12
    peak = PEAK_TFLOPS[cfg.precision]
    key = f"{phase}_{cfg.precision}_{cfg.name}"
    return {"kernel": kernel, "bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(ach / peak, 4), "traffic": _traffic(key), "flops_per_launch": flops,
            "avg_launch_ms": round(phase_ms[phase], 4)}


def fc1_roofline(cfg, phase_ms):
    # gate-up GEMM: 2 * R * H * (2I) flops
    return gemm_roofline(cfg, phase_ms, "fc1_gateup_swiglu", 4.0 * cfg.R * cfg.H * cfg.I,
                         "fwd_gemm_kernel (FC1 gate-up + ScaledSwiGLU*prob)")


def mem_bytes(cfg, split_sizes):
    """Algorithmic bytes per launch of the forward's memory-bound phases: read-once inputs plus
    written outputs plus index metadata."""
    R, H, I, E = cfg.R, cfg.H, cfg.I, cfg.E
    esz = 4 if cfg.x_dtype == "f32" else 2
    op = 1 + 1 / 32 if cfg.precision == "mxfp8" else 2
    if cfg.precision == "fp8":
        # bf16 rows written, then read by the amax and the quantize pass, codes written
        op = 2 + 2 + 2 + 1
    b = {"permute_rows": cfg.T * H * esz + R * H * op + R * 4}
    zsz = 2 if cfg.x_dtype == "bf16" else 4
    b["combine"] = R * H * zsz + cfg.T * H * esz + R * 4
    if cfg.precision == "mxfp8":
        nz = sum(1 for c in split_sizes if c > 0)
        b["quant_w1"] = nz * 2 * I * H * (2 + 1 + 1 / 32)
        b["quant_w2"] = nz * H * I * (2 + 1 + 1 / 32)
    if cfg.precision == "fp8":
        # two passes over every bf16 weight (amax, then quantize) and the codes written
        b["quant_w1"] = E * 2 * I * H * (2 + 2 + 1)
        b["quant_w2"] = E * H * I * (2 + 2 + 1)
    return b


def fwd_leg(cfg, steps, warmup, cold_steps=5, copy_ceiling=None):
    r = run_gpu(cfg, steps, warmup, cold_steps=cold_steps)
    ms = r["ms_per_step"]
    ph = r["phase_ms"]
    R, H, I = cfg.R, cfg.H, cfg.I
    mb = mem_bytes(cfg, r["split_sizes"])
    hbm = {k_: v / (ph[k_] * 1e-3) / 1e9 for k_, v in mb.items()}
    memory = {}
    for k_, v in mb.items():
        warm = r["stats"]["phase_ms"][k_]["median"]
        ent = {"bytes_per_launch": int(v), "warm_median_ms": warm, "warm_GBs": round(v / (warm * 1e-3) / 1e9, 1),
               "frac_of_8TBs_warm": round(v / (warm * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}
        if "cold" in r:
            cold = r["cold"]["phase_ms"][k_]["median"]
            ent.update({"cold_median_ms": cold, "cold_GBs": round(v / (cold * 1e-3) / 1e9, 1),
                        "frac_of_8TBs_cold": round(v / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
        if copy_ceiling:
            ent["frac_of_copy_warm"] = round(ent["warm_GBs"] / copy_ceiling[0], 3)
            if copy_ceiling[1]:
                ent["frac_of_copy64_warm"] = round(ent["warm_GBs"] / copy_ceiling[1], 3)
        memory[k_] = ent
    out = {
        "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "tflops": round(cfg.fwd_flops() / (ms * 1e-3) / 1e12, 1),
        "roofline": fc1_roofline(cfg, ph),
        "fc2_tflops": round(2.0 * R * H * I / (ph["fc2_down"] * 1e-3) / 1e12, 1),
        "hbm_GBs": {k_: round(v, 1) for k_, v in hbm.items()},
        "memory_kernels": memory,
        "phase_ms": {k_: round(v, 4) for k_, v in ph.items()},
        "stats": r["stats"],
        "split_sizes": r["split_sizes"],
        "tile_cycles": r["tile_cycles"],
    }
    if "cold" in r:
        out["cold"] = r["cold"]
    return r, out


def copy_leg(reps=10):
    """The practical HBM ceiling on this GPU: device-to-device copies (read + write), a read-only
    pass and a write-only fill of 64 MiB, 512 MiB and 2 GiB (64 MiB: a copy moving about as many
    bytes as one permute or combine launch), warm (back to back) and cold (a 1 GiB flush before
    each), HIP-event timed, median over reps.  GB/s count every byte read and written."""
    import torch
    fl = _flusher()
    res = {}
    for mib in (64, 512, 2048):
        n = mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        kinds = {"copy": (lambda: b.copy_(a), 2 * n * 4), "read": (lambda: a.sum(), n * 4),
                 "write": (lambda: b.fill_(2.0), n * 4)}
        for kind, (f, nbytes) in kinds.items():
            for cold in (False, True):
                f()
                torch.cuda.synchronize()
                ts = []
                for _ in range(reps):
                    if cold:
                        fl()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    f()
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1))
                med = _stats(ts)["median"]
                res[f"{kind}_{mib}MiB_{'cold' if cold else 'warm'}_GBs"] = round(nbytes / (med * 1e-3) / 1e9, 1)
        del a, b
    del fl
    torch.cuda.empty_cache()
    return res


def bwd_leg(cfg, steps, warmup, per_call_wt=False):
    r = run_gpu(cfg, steps, warmup, backward=True, per_call_wt=per_call_wt)
    ms = r["ms_per_step"]
    ph = r["phase_ms"]
    R, H, I = cfg.R, cfg.H, cfg.I
    gem = {"dgrad_fc2_swiglu_bwd": 2.0 * R * H * I, "wgrad_fc2": 2.0 * R * H * I,
           "dgrad_fc1": 4.0 * R * H * I, "wgrad_fc1": 4.0 * R * H * I}
    dom = max(gem, key=lambda k_: ph[k_])
    return {
        "workload": f"{cfg.name}: T={cfg.T} H={H} I={I} E={cfg.E} top-{cfg.k}, {cfg.precision} GEMM operands"
                    + (" (each quantized along its GEMM's K)" if cfg.precision == "mxfp8" else "") + ", dW in fp32",
        "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
        "tflops": round(cfg.bwd_flops() / (ms * 1e-3) / 1e12, 1),
        "roofline": gemm_roofline(cfg, ph, dom, gem[dom], f"bwd_gemm_kernel ({dom})"),
        "gemm_tflops": {k_: round(v / (ph[k_] * 1e-3) / 1e12, 1) for k_, v in gem.items()},
        "phase_ms": {k_: round(v, 4) for k_, v in ph.items()},
        "stats": r["stats"],
        # the forward of the same training step (saving for the backward; under MXFP8 it also
        # quantizes the weights along the backward's K) and the step's total
        "forward_with_save_ms": round(r["fwd_save"]["ms_per_step"], 4),
        "forward_with_save_phase_ms": {k_: round(v, 4) for k_, v in r["fwd_save"]["phase_ms"].items()},
        "train_step_ms": round(r["fwd_save"]["ms_per_step"] + ms, 4),
        "train_step_tokens_per_s": round(cfg.T / ((r["fwd_save"]["ms_per_step"] + ms) * 1e-3), 1),
        "tile_cycles": r["tile_cycles"],
    }


def router_leg(cfg, steps=20, warmup=5):
    """The fused router alone and fused with the permutation, on the workload's own logits
    (outputs and workspace allocated once; HIP-event timing on the current stream)."""
    import numpy as np
    import torch
    import mixture_experts_grouped_permute_amd as m
    from mixture_experts_grouped_permute_amd import _lib as L
    from moe_inputs import make_logits
    lib = m.load()
    dev = torch.device("cuda:0")
    T, E, k, H = cfg.T, cfg.E, cfg.k, cfg.H
    R = T * k
    lg = torch.from_numpy(make_logits(cfg).astype(np.float32)).to(dev)
    g = np.random.Generator(np.random.PCG64(cfg.seed))
    x = torch.from_numpy(g.standard_normal((T, H), dtype=np.float32)).to(torch.bfloat16).to(dev)
    i32 = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    idx, prob = i32(R), torch.empty(R, dtype=torch.float32, device=dev)
    split, offs, rid, src = i32(E), i32(E + 1), i32(R), i32(R)
    pperm = torch.empty(R, dtype=torch.float32, device=dev)
    mx = cfg.precision == "mxfp8"
    xp = torch.empty((R, H), dtype=torch.uint8 if mx else torch.bfloat16, device=dev)
    xs = torch.empty((R, H // 32), dtype=torch.uint8, device=dev) if mx else None
    ws = torch.empty(lib.moe_permute_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    pd = L.MOE_MXFP8_E4M3 if mx else L.MOE_BF16

    def route():
        L._check(lib.moe_route_topk(lg.data_ptr(), L.MOE_F32, T, E, k, idx.data_ptr(), prob.data_ptr(), st), "route")

    def route_permute():
        L._check(lib.moe_route_permute(lg.data_ptr(), L.MOE_F32, x.data_ptr(), L.MOE_BF16, T, H, E, k, pd,
                                       idx.data_ptr(), prob.data_ptr(), xp.data_ptr(), L._ptr(xs), split.data_ptr(),
                                       offs.data_ptr(), rid.data_ptr(), src.data_ptr(), pperm.data_ptr(),
                                       ws.data_ptr(), ws.numel(), st), "route_permute")

    def permute_only():
        L._check(lib.moe_permute(x.data_ptr(), L.MOE_BF16, T, H, idx.data_ptr(), prob.data_ptr(), k, E, pd,
                                 xp.data_ptr(), L._ptr(xs), split.data_ptr(), offs.data_ptr(), rid.data_ptr(),
                                 src.data_ptr(), pperm.data_ptr(), ws.data_ptr(), ws.numel(), st), "permute")

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            f()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    ms_route, ms_rp, ms_perm = timed(route), timed(route_permute), timed(permute_only)
    route_bytes = T * E * 4 + R * 8
    return {"route_us": round(ms_route * 1e3, 1), "route_hbm_GBs": round(route_bytes / (ms_route * 1e-3) / 1e9, 1),
            "route_permute_us": round(ms_rp * 1e3, 1),
            "route_then_permute_us": round((ms_route + ms_perm) * 1e3, 1)}


def loop_leg(cfg, steps=10, warmup=3):
    """Grouped forward against the per-expert loop of launches (host-side counts given), same
    inputs and workspace, HIP-event timing on the current stream."""
    import numpy as np
    import torch
    import mixture_experts_grouped_permute_amd as m
    from mixture_experts_grouped_permute_amd import _lib as L
    from moe_inputs import make_inputs
    lib = m.load()
    inp = make_inputs(cfg)
    d = inp.to("cuda:0")
    dev = d.x.device
    T, E, k, R = cfg.T, cfg.E, cfg.k, cfg.R
    perm = {n: torch.empty(sz, dtype=dt, device=dev) for n, sz, dt in
            (("split_sizes", E, torch.int32), ("offsets", E + 1, torch.int32), ("row_id_map", R, torch.int32),
             ("src_index", R, torch.int32), ("prob_perm", R, torch.float32))}
    out = torch.empty((T, cfg.H), dtype=d.x.dtype, device=dev)
    a, keep, _, _ = L._fwd_args(d.x, d.topk_idx, d.topk_prob, d.w1, d.w2, cfg.precision, out, perm, None)
    ws = torch.empty(lib.moe_grouped_mlp_fwd_workspace(ctypes.byref(a)), dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    counts = np.bincount(inp.topk_idx.numpy().ravel(), minlength=E)
    hc = (ctypes.c_int32 * E)(*[int(c) for c in counts])
    st = torch.cuda.current_stream(dev).cuda_stream

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            f()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps

    ms_g = timed(lambda: L._check(lib.moe_grouped_mlp_fwd(ctypes.byref(a), st), "grouped"))
    ms_l = timed(lambda: L._check(lib.moe_grouped_mlp_fwd_loop(ctypes.byref(a), hc, st), "loop"))
    del keep
    return {"grouped_ms": round(ms_g, 4), "loop_ms": round(ms_l, 4), "loop_over_grouped": round(ms_l / ms_g, 3),
            "experts_with_tokens": int((counts > 0).sum())}


def cpu_baseline(inp, cfg, tokens, min_seconds=12.0, max_passes=8):
    """The fp64 oracle on the first `tokens` tokens of the workload (its full expert weights),
    repeated until about min_seconds of CPU work have run."""
    from oracle import mlp
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    xs = inp.x[:tokens]
    idx = inp.topk_idx[:tokens].numpy()
    pr = inp.topk_prob[:tokens]
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        mlp.forward(xs, idx, pr, inp.w1, inp.w2, cfg.precision, cfg.x_dtype)
        dt += time.perf_counter() - t0
        passes += 1
    return {"value": round(passes * tokens / dt, 2), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": model, "blas_threads": int(threads),
            "sample": f"{passes} passes over the first {tokens} of {cfg.T} tokens of the same workload, all "
                      f"{cfg.E} experts' full weights (fp64 numpy per-expert loop, {threads} BLAS threads on "
                      f"{cores} cores available to the process), {dt:.1f} s in total"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-mxfp8", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-tile-stats", action="store_true",
                    help="skip the untimed call with the GEMM cycle counters on (keeps profiler pass counts)")
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--legs", default="copy,bf16,mxfp8,mxfp8_finegrained,fp8,backward,backward_mxfp8,router,loop,"
                                      "mfma_probe",
                    help="comma list of copy, bf16, mxfp8, mxfp8_finegrained, fp8, backward, backward_mxfp8, router, "
                         "loop, mfma_probe (bf16 always runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 5 times (counter calibration)")
    ap.add_argument("--lib-gemm-probe", action="store_true",
                    help="only time torch.matmul on the gate-up projection's shape as one dense bf16 GEMM "
                         "(M = T*k = 8192, K = 4096, N = 2*14336), a reference for the MFMA counters")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only run the library's MFMA issue-rate probe (moe_mfma_probe): cycles per MFMA of "
                         "the bf16 and the E4M3 MFMA-scale instruction on all 1024 SIMDs, and the clock")
    ap.add_argument("--load-probe", action="store_true",
                    help="only run the library's LDS fill-rate probe (moe_load_probe) on its four access patterns")
    args = ap.parse_args()
    global TILE_STATS
    TILE_STATS = not args.no_tile_stats
    if args.lib_gemm_probe:
        import torch
        g = torch.Generator(device="cuda:0").manual_seed(0)
        a = torch.randn(8192, 4096, device="cuda:0", generator=g).to(torch.bfloat16)
        b = (torch.randn(4096, 28672, device="cuda:0", generator=g) * 0.02).to(torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, b)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        med = _stats(ts)["median"]
        flops = 2.0 * 8192 * 4096 * 28672
        print(json.dumps({"lib_gemm_probe": "torch.matmul bf16 8192x4096 @ 4096x28672", "median_ms": med,
                          "tflops": round(flops / (med * 1e-3) / 1e12, 1)}), flush=True)
        return
    if args.load_probe:
        import torch
        import mixture_experts_grouped_permute_amd as m
        buf = torch.zeros(m.load().moe_load_probe_bytes(), dtype=torch.uint8, device="cuda:0")
        for pat in range(4):
            print(json.dumps({"load_probe": m.load_probe(pat, buf=buf)}), flush=True)
        return
    if args.mfma_probe:
        import mixture_experts_grouped_permute_amd as m
        for kind in (2, 3, 0, 4, 1):
            print(json.dumps({"mfma_probe": m.mfma_probe(kind)}), flush=True)
        return
    if args.copy_probe:
        import torch
        src = torch.empty(args.copy_probe // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "launches": 5}), flush=True)
        return
    legs = set(x.strip() for x in args.legs.split(",") if x.strip())
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this layer runs unsharded on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    from moe_inputs import get_config

    copy = None
    if "copy" in legs:
        _log("timing the copy ceiling")
        copy = copy_leg()
    ceiling = (copy["copy_2048MiB_warm_GBs"], copy["copy_64MiB_warm_GBs"]) if copy else None
    cfg = get_config(2)
    r, leg = fwd_leg(cfg, args.steps, args.warmup, copy_ceiling=ceiling)
    ms = leg["ms_per_step"]
    line = {
        "metric": METRIC, "value": leg["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} top-{cfg.k}, "
                               f"bf16 operands, fp32 accumulation, N(0,1) router logits",
                   "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "top_k": cfg.k, "parallelism": "none (1 GPU)"},
        "tflops": leg["tflops"], "roofline": leg["roofline"],
        "fc2_tflops": leg["fc2_tflops"], "hbm_GBs": leg["hbm_GBs"],
        "phase_ms": leg["phase_ms"], "stats": leg["stats"], "cold": leg.get("cold"),
        "memory_kernels": leg["memory_kernels"], "split_sizes": leg["split_sizes"],
        "tile_cycles": leg["tile_cycles"],
    }
    if copy:
        line["copy_ceiling"] = copy
    if not args.no_cpu_baseline:
        _log(f"timing the CPU oracle on {args.cpu_tokens} tokens")
        line["cpu_baseline"] = cpu_baseline(r["inputs"], cfg, args.cpu_tokens)
    del r
    import torch
    if not args.no_mxfp8:
        for key, ci in (("mxfp8", 3), ("mxfp8_finegrained", 5)):
            if key not in legs:
                continue
            torch.cuda.empty_cache()
            c = get_config(ci)
            rr, lg = fwd_leg(c, max(2, args.steps // 2), max(1, args.warmup // 2), copy_ceiling=ceiling)
            del rr
            torch.cuda.empty_cache()
            rc = run_gpu(c, max(2, args.steps // 2), max(1, args.warmup // 2), cached=True)
            lg["cached_weights"] = {"ms_per_step": round(rc["ms_per_step"], 4),
                                    "value": round(c.T / (rc["ms_per_step"] * 1e-3), 1), "unit": "tokens/s",
                                    "note": "MXFP8 weights quantized once and passed in (not per call)"}
            del rc
            lg["workload"] = (f"{c.name}: T={c.T} H={c.H} I={c.I} E={c.E} top-{c.k}, MXFP8 both GEMMs, "
                              f"Zipf({c.zipf_s}) routing" + (f", expert {c.zero_expert} empty" if c.zero_expert is not None else "")
                              + ", weights quantized per call")
            line[key] = lg
        if "fp8" in legs:
            torch.cuda.empty_cache()
            c = get_config(3).with_(precision="fp8")
            rr, lg = fwd_leg(c, max(2, args.steps // 2), max(1, args.warmup // 2), copy_ceiling=ceiling)
            del rr
            torch.cuda.empty_cache()
            rc = run_gpu(c, max(2, args.steps // 2), max(1, args.warmup // 2), cached=True)
            lg["cached_weights"] = {"ms_per_step": round(rc["ms_per_step"], 4),
                                    "value": round(c.T / (rc["ms_per_step"] * 1e-3), 1), "unit": "tokens/s",
                                    "note": "per-tensor FP8 weights quantized once and passed in (not per call)"}
            del rc
            lg["workload"] = (f"{c.name} shape and routing: T={c.T} H={c.H} I={c.I} E={c.E} top-{c.k}, "
                              f"per-tensor-scaled FP8 (E4M3, one fp32 scale per operand tensor) both GEMMs, "
                              f"weights quantized per call; fc1_gateup_swiglu includes h's amax and quantize "
                              f"passes, permute_rows those of X_perm")
            line["fp8_tensor"] = lg
    if "loop" in legs:
        torch.cuda.empty_cache()
        line["loop_vs_grouped"] = {c.name: loop_leg(c) for c in (get_config(2), get_config(5))}
    if "router" in legs:
        line["router"] = {c.name: router_leg(c) for c in (get_config(2), get_config(5))}
    if not args.no_backward and "backward" in legs:
        torch.cuda.empty_cache()
        line["backward_bf16"] = bwd_leg(get_config(4), max(2, args.steps // 2), max(1, args.warmup // 2))
    if not args.no_backward and "backward_mxfp8" in legs:
        # the MXFP8 backward on the same workload (its forward run with MXFP8 too)
        torch.cuda.empty_cache()
        line["backward_mxfp8"] = bwd_leg(get_config(4).with_(precision="mxfp8"), max(2, args.steps // 2),
                                         max(1, args.warmup // 2))
        # the same step with the backward quantizing W1, W2 along its K itself (the forward quantizing
        # only its own copy)
        torch.cuda.empty_cache()
        rc = bwd_leg(get_config(4).with_(precision="mxfp8"), max(2, args.steps // 2), max(1, args.warmup // 2),
                     per_call_wt=True)
        line["backward_mxfp8"]["per_call_weights"] = {
            k_: rc[k_] for k_ in ("ms_per_step", "value", "phase_ms", "forward_with_save_ms", "train_step_ms")}
    if "mfma_probe" in legs:
        # after every timed region: the matrix cores' own rate with GEMM-like random operands, beside
        # the published peak of each roofline (bf16 for peak 2500, E4M3 otherwise)
        annotate_rooflines(line)
    print(json.dumps(line), flush=True)


def annotate_rooflines(line):
    """Add the library MFMA probe's random-operand ceiling (kinds 3 and 4: 4 A x 4 B pseudo-random
    fragments, no memory traffic) to every roofline object of the line, with achieved / ceiling."""
    import mixture_experts_grouped_permute_amd as m
    ceil = {2500.0: m.mfma_probe(3, iters=1000)["tflops"], 5000.0: m.mfma_probe(4, iters=1000)["tflops"]}
    objs = [line.get("roofline")] + [v.get("roofline") for v in line.values() if isinstance(v, dict)]
    for rf in objs:
        if not rf or rf.get("unit") != "TFLOP/s" or rf.get("peak") not in ceil:
            continue
        c = ceil[rf["peak"]]
        rf["mfma_probe_ceiling"] = c
        rf["frac_of_mfma_probe"] = round(rf["achieved"] / c, 4)


if __name__ == "__main__":
    main()
