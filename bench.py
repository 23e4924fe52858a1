"""Layer-quantization throughput of the KronQ per-layer solver on one MI355X.

One step = the whole per-layer path on device-resident inputs (X, W, H_G, signs):
  H_X accumulation, sensitivity, input rotation, H_G^{1/2} (+ inverse), output transform,
  damped inverse factor, GPTQ sweep with packing.
Workload: 4096 x 4096 layer, 65536 bf16 calibration tokens, full H_G, 3-bit asymmetric, group 128
(synthetic, seeded; stands in for the LLaMA-2-7B q_proj layer the KronQ pages quantize).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK = {"hbm": 8.0e12, "fp32_mfma": 157.3e12, "fp64_alu": 78.6e12, "bf16_mfma": 2.5e15}
DB_TOL = 1e-8      # stopping bound of the Denman-Beavers square root (same constant as the library)
DB_NS_MAX = 8e-5   # bound under which the library's last step is the Newton-Schulz step (same constant)


def db_plan(blocks) -> tuple:
    """Steps the library's square root takes for the given full H_G blocks, and whether the last is the
    Newton-Schulz step: each block's x-interval starts at [sqrt(1/||A^-1||_F), sqrt(||A||_F)], its bound
    b follows b <- (sqrt(b) + 1/sqrt(b)) / 2 after the first step, and the loop stops once b - 1 < DB_TOL
    for every block; the last step is replaced when every bound before it is within DB_NS_MAX of 1."""
    firsts = []
    for HG in blocks:
        A = HG.astype(np.float64)
        r = math.sqrt(np.linalg.norm(A) * np.linalg.norm(np.linalg.inv(A)))
        firsts.append(0.5 * (math.sqrt(r) + 1.0 / math.sqrt(r)))

    def after(b, k):   # bound after k steps
        for _ in range(k - 1):
            b = 0.5 * (math.sqrt(b) + 1.0 / math.sqrt(b))
        return b

    need = 1
    for b in firsts:
        k = 1
        while after(b, k) - 1.0 >= DB_TOL and k < 7:
            k += 1
        need = max(need, k)
    ns = need >= 2 and all(after(b, need - 1) - 1.0 <= DB_NS_MAX for b in firsts)
    return need, ns


def algorithmic_work(sp, plan: tuple) -> dict:
    """Per-phase algorithmic FLOP / bytes of one layer: what the method must compute or move.

    hessian: the symmetric product n i (i+1); rotate_in: W read (bf16/fp32) and W' written (fp32),
    H_X read and written twice (fp64, rows then columns); hg_sqrt (full H_G): one SPD inverse of n^3
    FLOP in the first Denman-Beavers step and two in every later one, and for a Newton-Schulz last
    step the fp64 product E = I - Z Y (lower triangle, n^3; its fp32 product Y E / 2, 2 n^3 on the
    matrix cores, is not counted against the fp64 peak); rotate_out: 8 B per weight for
    the V pass plus the 2 o^2 i FLOP of S W' (full H_G); cholinv: 2 i^3 / 3; quantize: the sweep's
    bytes (W'' read and Q'' written, codes, grid parameters, R) and the trailing-update FLOP."""
    o, i, n, b, g = sp.o, sp.i, sp.n, sp.bits, sp.group
    xb = 2 if sp.x_dtype == "bf16" else 4
    wb = 2 if sp.w_dtype == "bf16" else 4
    full = sp.hg_form == "full"
    need, ns = plan
    dbs = need - 1 if ns else need
    unit = o ** 3 if full else ((o // sp.hg_blk) * sp.hg_blk ** 3 if sp.hg_form == "block" else 0)
    return {
        "hessian": {"flop": n * i * (i + 1), "bytes": n * i * xb + 8 * i * i, "peak": "bf16_mfma"},
        "rotate_in": {"bytes": o * i * (wb + 4) + 32 * i * i, "peak": "hbm"},
        "hg_sqrt": {"flop": ((2 * dbs - 1) + (1 if ns else 0)) * unit if sp.hg_form != "diag" else 0,
                    "peak": "fp64_alu"},
        "rotate_out": ({"flop": 2 * o * o * i, "peak": "fp32_mfma"} if full else {"bytes": 8 * o * i, "peak": "hbm"}),
        "cholinv": {"flop": 2 * i ** 3 // 3, "peak": "fp64_alu"},
        "quantize": {"bytes": int((8 + b / 8 + (8 / g if g else 0)) * o * i + 2 * i * i),
                     "flop": o * i * (i - 128), "peak": "hbm", "flop_peak": "fp32_mfma"},
    }


def sources_digest() -> str:
    """sha256 over the library's HIP sources, to tie a committed counter measurement to a build."""
    import hashlib
    import glob
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "post_quantization_03_amd", "csrc", "*"))):
        if os.path.basename(f) == "probe.hip":   # the throughput probes are not part of the library
            continue
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(phase: str):
    """HBM bytes per call of a phase from the committed rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
    summary (profiles/<phase>_c2_traffic.md), or None when the sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{phase}_c2_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":", 1)[0].strip() in ("sources-sha256", "bytes-per-call"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("sources-sha256") != sources_digest() or "bytes-per-call" not in vals:
        return None
    return int(vals["bytes-per-call"])


def roofline_of(name: str, wk: dict, ms: float) -> dict:
    """The phase's roofline: its algorithmic work over its time against the peak of the resource that
    bounds it. A phase with both bytes and FLOP (the sweep: HBM streaming and the trailing-update
    products) is bound by whichever needs the longer time at its peak."""
    pk = wk["peak"]
    if pk == "hbm" and wk.get("flop_peak") and wk["flop"] / PEAK[wk["flop_peak"]] > wk["bytes"] / PEAK["hbm"]:
        pk = wk["flop_peak"]
    if pk == "hbm":
        ach = wk["bytes"] / (ms / 1e3)
        return {"bound": "hbm", "kernel": name, "achieved": round(ach / 1e9, 2), "peak": PEAK["hbm"] / 1e9,
                "unit": "GB/s", "frac": round(ach / PEAK["hbm"], 4), "traffic": None}
    ach = wk["flop"] / (ms / 1e3)
    bound = "alu" if pk == "fp64_alu" else "mfma"
    return {"bound": bound, "kernel": name, "achieved": round(ach / 1e12, 3), "peak": PEAK[pk] / 1e12,
            "unit": "TFLOP/s", "frac": round(ach / PEAK[pk], 4), "traffic": None}


def run_gpu(sp, steps: int, warmup: int, phases: bool):
    import torch

    from post_quantization_03_amd import _lib as K
    from post_quantization_03_amd.layer import LayerCfg, quantize_layer, workspace_bytes

    dev = torch.device("cuda:0")
    t0 = time.time()
    d = synth.layer_inputs(sp)
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def to(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    iters = db_plan([d["HG"]]) if sp.hg_form == "full" else (
        db_plan(list(d["HG"])) if sp.hg_form == "block" else (0, False))
    X, W, HG = to(d["X"], sp.x_dtype), to(d["W"], sp.w_dtype), to(d["HG"], "f32")
    s, t = to(d["s"], "i8"), to(d["t"], "i8")
    del d
    cfg = LayerCfg(bits=sp.bits, group=sp.group, damp=sp.damp, form=sp.hg_form,
                   blk=sp.hg_blk if sp.hg_form == "block" else 0)
    xdt = K.KQ_BF16 if sp.x_dtype == "bf16" else K.KQ_F32
    ws = torch.empty(workspace_bytes(sp.o, sp.i, sp.n, xdt, cfg), dtype=torch.uint8, device=dev)

    def step():
        return quantize_layer(X, W, HG, s, t, cfg, ws=ws)

    for k in range(warmup):
        out = step()
        torch.cuda.synchronize()
        print(f"# warmup {k + 1}/{warmup} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps):
        out = step()
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    info = out["info"].cpu().tolist()
    if info != [0, 0]:
        raise RuntimeError(f"factorisation failed: info={info}")
    ms = 1e3 * t_total / steps
    print(f"# timed {steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    ph, ms_cached = None, None
    if phases:
        ph = phase_times(sp, X, W, HG, s, t, cfg, ws)
        # the same step with S = H_G^1/2 already on the device (a layer whose H_G factor is reused)
        Sc = (out["S"], None)
        quantize_layer(X, W, HG, s, t, cfg, ws=ws, S_cached=Sc)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(steps):
            quantize_layer(X, W, HG, s, t, cfg, ws=ws, S_cached=Sc)
        torch.cuda.synchronize()
        ms_cached = 1e3 * (time.perf_counter() - t_start) / steps
    mv = matvec_times(sp, out, HG, s, t, cfg) if phases else None
    return ms, ph, out, iters, mv, ms_cached


def phase_times(sp, X, W, HG, s, t, cfg, ws, reps: int = 3) -> dict:
    """Median per-phase time (ms) of the same calls, with HIP events on the stream they run on."""
    import torch

    from post_quantization_03_amd import _lib as K
    from post_quantization_03_amd.layer import hg_factor_shape

    dev = X.device
    o, i, n = sp.o, sp.i, sp.n
    f32 = dict(dtype=torch.float32, device=dev)
    H = torch.empty((i, i), dtype=torch.float64, device=dev)
    W2 = torch.empty((o, i), **f32)
    S = torch.empty(hg_factor_shape(o, cfg), **f32)
    R = torch.empty((i, i), **f32)
    info = torch.zeros(2, dtype=torch.int32, device=dev)
    score = torch.empty(1, dtype=torch.float64, device=dev)
    ng = i // cfg.group if cfg.group else 1
    codes = torch.empty((o, i * cfg.bits // 32), dtype=torch.int32, device=dev)
    scale = torch.empty((o, ng), **f32)
    offset = torch.empty((o, ng), **f32)
    rl = torch.empty((o,), **f32)
    calls = [
        ("hessian", lambda: K.kq_hessian_accum(X, H, 1.0 / n, 0.0, ws)),
        ("sensitivity", lambda: K.kq_sensitivity(H, HG, cfg.form, o, cfg.blk, score)),
        ("rotate_in", lambda: K.kq_rotate_in(W, W2, H, s, ws)),
        ("hg_sqrt", lambda: K.kq_hg_sqrt(HG, cfg.form, o, cfg.blk, S, None, info[0:1], ws)),
        ("rotate_out", lambda: K.kq_rotate_out(W2, S, cfg.form, cfg.blk, t, ws)),
        ("cholinv", lambda: K.kq_cholinv(H, cfg.damp, R, info[1:2], ws)),
        ("quantize", lambda: K.kq_quantize_layer(W2, R, cfg.bits, cfg.group, cfg.block, codes, scale, offset, rl, ws)),
    ]
    res = {name: [] for name, _ in calls}
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
        ev[0].record()
        for k, (name, fn) in enumerate(calls):
            fn()
            ev[k + 1].record()
        torch.cuda.synchronize()
        for k, (name, _) in enumerate(calls):
            res[name].append(ev[k].elapsed_time(ev[k + 1]))
    out = {k: float(np.median(v)) for k, v in res.items()}
    out["_chain"] = sweep_chain(sp, W2, R, cfg, reps)
    return out


def sweep_chain(sp, W2, R, cfg, reps: int = 3) -> float:
    """The sweep's dependent chain (ms): kq_quantize_layer on 16 rows alone, i.e. one work-group per
    128-column block, so the time is the i dependent column steps of a row plus what separates the
    blocks (launches, the lazy trailing updates). No schedule of the sweep can finish a row sooner."""
    import torch

    from post_quantization_03_amd import _lib as K

    dev = W2.device
    rows = 16
    Wr = W2[:rows].clone()
    ng = sp.i // cfg.group if cfg.group else 1
    codes = torch.empty((rows, sp.i * cfg.bits // 32), dtype=torch.int32, device=dev)
    scale = torch.empty((rows, ng), dtype=torch.float32, device=dev)
    offset = torch.empty((rows, ng), dtype=torch.float32, device=dev)
    rl = torch.empty((rows,), dtype=torch.float32, device=dev)
    ws = torch.empty(max(K.kq_workspace_bytes("quantize", rows, sp.i), 256), dtype=torch.uint8, device=dev)
    times = []
    for _ in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        K.kq_quantize_layer(Wr, R, cfg.bits, cfg.group, cfg.block, codes, scale, offset, rl, ws)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return float(np.median(times[1:]))


def matvec_times(sp, out, HG, s, t, cfg, reps: int = 200) -> dict:
    """Inference-side product y = W^ x from the packed codes this step wrote (kq_matvec_quantized:
    x' = U^T x, the dequantizing product, then S^{-1} V^T), for 1 and 8 tokens. Time per call from HIP
    events around `reps` calls replayed from a HIP graph (and, as `us_per_call_eager`, around `reps`
    back-to-back calls from Python, which the host's launch cost bounds); algorithmic bytes = the
    packed codes, the group scales and offsets, S^{-1} in its storage form, the signs, x and y."""
    import torch

    from post_quantization_03_amd import _lib as K

    dev = HG.device
    o, i = sp.o, sp.i
    S = torch.empty_like(out["S"])
    Sinv = torch.empty_like(out["S"])
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(K.kq_workspace_bytes("hg_sqrt", o, 0, form=cfg.form, blk=cfg.blk),
                         K.kq_workspace_bytes("matvec", o, i, 8, form=cfg.form, blk=cfg.blk)), dtype=torch.uint8,
                     device=dev)
    K.kq_hg_sqrt(HG, cfg.form, o, cfg.blk, S, Sinv, info, ws)
    res = time_matvec(sp, cfg, out["codes"], out["scale"], out["offset"], s, t, Sinv, ws, reps)
    if int(info.item()) != 0:
        raise RuntimeError("square root for the product did not converge")
    return res


def time_matvec(sp, cfg, codes, scale, offset, s, t, Sinv, ws, reps: int = 200) -> dict:
    import torch

    from post_quantization_03_amd import _lib as K

    dev = codes.device
    o, i, b = sp.o, sp.i, sp.bits
    res = {}
    for nt in (1, 8):
        x = torch.randn((nt, i), dtype=torch.float32, device=dev)
        y = torch.empty((nt, o), dtype=torch.float32, device=dev)

        def call():
            K.kq_matvec_quantized(codes, scale, offset, o, i, b, cfg.group, s, t, Sinv, cfg.form, cfg.blk, x, y, ws)

        def timed(fn, n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        us_eager = 1e3 * timed(call, reps)
        # the same call captured once in a HIP graph: replays show the device time without the
        # host-side cost of each launch (a decode loop would replay it the same way)
        per_graph = 20
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for _ in range(per_graph):
                    call()
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        us = 1e3 * timed(g.replay, max(1, reps // per_graph)) / per_graph
        nbytes = (codes.numel() * 4 + (scale.numel() + offset.numel()) * 4 + Sinv.numel() * 4 + i + o
                  + 4 * nt * (i + o))
        ach = nbytes / (us / 1e6)
        res[f"nt{nt}"] = {"us_per_call": round(us, 2), "us_per_call_eager": round(us_eager, 2), "bytes": int(nbytes),
                          "achieved_GBps": round(ach / 1e9, 1), "frac_hbm": round(ach / PEAK["hbm"], 4)}
    return res


def matvec_only(sp) -> dict:
    """The inference-side product alone on the workload's layer shape and code layout: random packed
    words (every word is a valid code stream), group scales and offsets, signs, and S^{-1} in the
    workload's storage form (a positive diagonal, identity blocks or the identity), all device-resident."""
    import torch

    from post_quantization_03_amd import _lib as K
    from post_quantization_03_amd.layer import LayerCfg

    dev = torch.device("cuda:0")
    cfg = LayerCfg(bits=sp.bits, group=sp.group, damp=sp.damp, form=sp.hg_form,
                   blk=sp.hg_blk if sp.hg_form == "block" else 0)
    g = torch.Generator(device=dev)
    g.manual_seed(sp.o * 7 + sp.i)
    o, i, b = sp.o, sp.i, sp.bits
    ng = i // sp.group if sp.group else 1
    codes = torch.randint(-2 ** 31, 2 ** 31 - 1, (o, i * b // 32), dtype=torch.int32, device=dev, generator=g)
    scale = torch.rand((o, ng), device=dev, generator=g) * 0.01
    offset = -scale * 2 ** (b - 1)
    s = (torch.randint(0, 2, (i,), device=dev, generator=g) * 2 - 1).to(torch.int8)
    t = (torch.randint(0, 2, (o,), device=dev, generator=g) * 2 - 1).to(torch.int8)
    if cfg.form == "diag":
        Sinv = torch.rand(o, device=dev, generator=g) + 0.5
    elif cfg.form == "block":
        Sinv = torch.eye(cfg.blk, device=dev).repeat(o // cfg.blk, 1, 1).contiguous()
    else:
        Sinv = torch.eye(o, device=dev)
    ws = torch.empty(K.kq_workspace_bytes("matvec", o, i, 8, form=cfg.form, blk=cfg.blk), dtype=torch.uint8,
                     device=dev)
    return time_matvec(sp, cfg, codes, scale, offset, s, t, Sinv, ws)


def hg_variants(sp, ranks=(64, 256, 1024), q: int = 2) -> dict:
    """Effect of the H_G preparation on the layer: H_G streamed from the gradient rows
    (kq_hessian_accum on G), then quantized with the output-side root taken from the exact H_G, its
    128-block diagonal, its diagonal, the low-rank-plus-isotropic approximation of rank k built from
    G alone (kq_hg_lowrank), and no H_G at all (S = I). Every variant is scored with the exact
    K-FAC loss tr(H_G dW H_X dW^T) in the original coordinates (kq_kfac_loss); prep_ms is the time of
    forming S and S^{-1} (HIP events on the stream the calls run on)."""
    import torch

    from post_quantization_03_amd import _lib as K
    from post_quantization_03_amd.layer import LayerCfg

    if sp.hg_form != "full":
        raise ValueError("the variants start from a full H_G")
    dev = torch.device("cuda:0")
    d = synth.layer_inputs(sp)
    G = torch.from_numpy(synth.gen_G(sp)).to(dev)

    def to(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    X, W = to(d["X"], sp.x_dtype), to(d["W"], sp.w_dtype)
    s, t = to(d["s"], "i8"), to(d["t"], "i8")
    del d
    o, i, n, ng = sp.o, sp.i, sp.n, sp.hg_ng
    f32, f64 = dict(dtype=torch.float32, device=dev), dict(dtype=torch.float64, device=dev)
    cfg = LayerCfg(bits=sp.bits, group=sp.group, damp=sp.damp, form="full", blk=0)
    xdt = K.KQ_BF16 if sp.x_dtype == "bf16" else K.KQ_F32
    kmax = max(ranks)
    ws = torch.empty(max(K.kq_workspace_bytes(op, o, i, n, xdt, sp.bits, sp.group, form, 128)
                         for op in ("hessian", "rotate_in", "hg_sqrt", "rotate_out", "cholinv", "quantize",
                                    "unrotate", "kfac_loss") for form in ("full", "block", "diag")),
                     dtype=torch.uint8, device=dev)
    ws_g = torch.empty(max(K.kq_workspace_bytes("hessian", 0, o, ng, K.KQ_F32),
                           K.kq_workspace_bytes("hg_lowrank", o, kmax, ng)), dtype=torch.uint8, device=dev)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)
    # shared by every variant: H_X, the input rotation, the damped factor
    HX = torch.empty((i, i), **f64)
    K.kq_hessian_accum(X, HX, 1.0 / n, 0.0, ws)
    HX2 = HX.clone()
    W1 = torch.empty((o, i), **f32)
    K.kq_rotate_in(W, W1, HX2, s, ws)
    R = torch.empty((i, i), **f32)
    info = torch.zeros(4, dtype=torch.int32, device=dev)
    K.kq_cholinv(HX2, sp.damp, R, info[0:1], ws)
    # H_G streamed from the gradient rows, then its storage forms
    HG64 = torch.empty((o, o), **f64)
    stream_ms = timed(lambda: K.kq_hessian_accum(G, HG64, 1.0 / ng, 0.0, ws_g))
    HGf = torch.empty((o, o), **f32)
    K.kq_hg_extract(HG64, "full", 0, HGf)
    HGb = torch.empty((o // 128, 128, 128), **f32)
    K.kq_hg_extract(HG64, "block", 128, HGb)
    HGd = torch.empty((o,), **f32)
    K.kq_hg_extract(HG64, "diag", 0, HGd)
    ng_ = i // sp.group if sp.group else 1
    codes = torch.empty((o, i * sp.bits // 32), dtype=torch.int32, device=dev)
    scale, offset = torch.empty((o, ng_), **f32), torch.empty((o, ng_), **f32)
    loss = torch.empty(1, **f64)

    def run(form, blk, S, Sinv):
        W2 = W1.clone()
        K.kq_rotate_out(W2, S, form, blk, t, ws)
        K.kq_quantize_layer(W2, R, sp.bits, sp.group, 128, codes, scale, offset, None, ws)
        What = torch.empty((o, i), **f32)
        K.kq_unrotate(W2, s, t, Sinv, form, blk, What, ws)
        K.kq_kfac_loss(W, What, HX, HGf, "full", 0, loss, ws)
        torch.cuda.synchronize()
        return float(loss.item())
    out = {}
    for name, form, blk, HGv in (("full", "full", 0, HGf), ("block128", "block", 128, HGb), ("diag", "diag", 0, HGd)):
        S, Si = torch.empty_like(HGv), torch.empty_like(HGv)
        ms = timed(lambda: K.kq_hg_sqrt(HGv, form, o, blk, S, Si, info[1:2], ws))
        out[name] = {"prep_ms": round(ms, 3), "kfac_loss": run(form, blk, S, Si), "info": int(info[1].item())}
    for k in ranks:
        omega = torch.from_numpy(synth.gen_omega(sp, k)).to(dev)
        S, Si = torch.empty((o, o), **f32), torch.empty((o, o), **f32)
        sig = torch.empty(2, **f64)
        ms = timed(lambda: K.kq_hg_lowrank(G, k, q, omega, S, Si, None, sig, info[2:3], ws_g))
        out[f"lowrank{k}"] = {"prep_ms": round(ms, 3), "kfac_loss": run("full", 0, S, Si), "info": int(info[2].item()),
                              "sigma": float(sig[0].item())}
    ones = torch.ones((o,), **f32)
    out["identity"] = {"prep_ms": 0.0, "kfac_loss": run("diag", 0, ones, ones), "info": 0}
    base = out["full"]["kfac_loss"]
    for v in out.values():
        v["loss_vs_full"] = round(v["kfac_loss"] / base, 5)
    return {"workload": sp.name, "gradient_rows": ng, "power_steps": q, "streamed_hg_ms": round(stream_ms, 3),
            "hg_variants": out}


def solver_variants(sp, candidates: int = 500, reps: int = 3) -> dict:
    """The layer with the solver variants the pages describe for a related method: grids chosen by a
    Hessian-aware search over `candidates` scales, and 128-column blocks swept in descending trace of
    H_X'. Per variant: median time of the whole layer step (HIP events), and the exact K-FAC loss
    tr(H_G dW H_X dW^T) of its result relative to the plain solver's."""
    import dataclasses

    import torch

    from post_quantization_03_amd import _lib as K
    from post_quantization_03_amd.layer import LayerCfg, quantize_layer, workspace_bytes

    dev = torch.device("cuda:0")
    d = synth.layer_inputs(sp)

    def to(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    X, W, HG = to(d["X"], sp.x_dtype), to(d["W"], sp.w_dtype), to(d["HG"], "f32")
    s, t = to(d["s"], "i8"), to(d["t"], "i8")
    del d
    o, i, n = sp.o, sp.i, sp.n
    xdt = K.KQ_BF16 if sp.x_dtype == "bf16" else K.KQ_F32
    base = LayerCfg(bits=sp.bits, group=sp.group, damp=sp.damp, form=sp.hg_form,
                    blk=sp.hg_blk if sp.hg_form == "block" else 0)
    ws = torch.empty(max(workspace_bytes(o, i, n, xdt, base, verify=True),
                         K.kq_workspace_bytes("kfac_loss", o, i, form=base.form, blk=base.blk)),
                     dtype=torch.uint8, device=dev)
    HX = torch.empty((i, i), dtype=torch.float64, device=dev)
    K.kq_hessian_accum(X, HX, 1.0 / n, 0.0, ws)
    Sc = torch.empty((o, o) if base.form == "full" else HG.shape, dtype=torch.float32, device=dev)
    Sic = torch.empty_like(Sc)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    K.kq_hg_sqrt(HG, base.form, o, base.blk, Sc, Sic, info, ws)   # S cached: the variants differ after it
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    out = {}
    for name, kw in (("plain", {}), (f"search{candidates}", {"search": candidates}), ("trace_order", {"order": "trace"}),
                     (f"search{candidates}+trace_order", {"search": candidates, "order": "trace"})):
        cfg = dataclasses.replace(base, **kw)
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            r = quantize_layer(X, W, HG, s, t, cfg, ws=ws, S_cached=(Sc, Sic), verify=True)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        K.kq_kfac_loss(W, r["What"], HX, HG, base.form, base.blk, loss, ws)
        torch.cuda.synchronize()
        out[name] = {"layer_ms_S_cached": round(float(np.median(times)), 3), "kfac_loss": float(loss.item()),
                     "info": host_list(r["info"])}
    ref = out["plain"]["kfac_loss"]
    for v in out.values():
        v["loss_vs_plain"] = round(v["kfac_loss"] / ref, 5)
    return {"workload": sp.name, "variants": out}


def drift_study(sp, rel: float = 0.05, reps: int = 3) -> dict:
    """Input-drift correction on the workload's layer: the inputs drift by `rel` of each channel's
    scale (synth.gen_X_drift). Solvers: GPTQ on the clean H_X (target W), GPTQ on the drifted H~
    (target W), and the drift-corrected solver (target W* = W C (H~ + lambda I)^{-1} with H~). Each is
    scored by tr(H_G (W^ - W*) H~ (W^ - W*)^T), the part of the output error on the drifted inputs,
    tr(H_G (W^ X~^T - W X^T)(...)^T) / n, that depends on W^ (kq_kfac_loss with W* and H~), and
    timed as a whole layer step with S cached (HIP events, median)."""
    import torch

    from post_quantization_03_amd import _lib as K
    from post_quantization_03_amd.layer import LayerCfg, quantize_layer, workspace_bytes

    dev = torch.device("cuda:0")
    d = synth.layer_inputs(sp)

    def to(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    X, W, HG = to(d["X"], sp.x_dtype), to(d["W"], sp.w_dtype), to(d["HG"], "f32")
    Xt = to(synth.gen_X_drift(sp, rel=rel), sp.x_dtype)
    s, t = to(d["s"], "i8"), to(d["t"], "i8")
    del d
    o, i, n = sp.o, sp.i, sp.n
    xdt = K.KQ_BF16 if sp.x_dtype == "bf16" else K.KQ_F32
    cfg = LayerCfg(bits=sp.bits, group=sp.group, damp=sp.damp, form=sp.hg_form,
                   blk=sp.hg_blk if sp.hg_form == "block" else 0)
    ws = torch.empty(max(workspace_bytes(o, i, n, xdt, cfg, verify=True),
                         K.kq_workspace_bytes("kfac_loss", o, i, form=cfg.form, blk=cfg.blk),
                         K.kq_workspace_bytes("cross", 0, i, n), K.kq_workspace_bytes("drift", o, i)),
                     dtype=torch.uint8, device=dev)
    Ht = torch.empty((i, i), dtype=torch.float64, device=dev)
    K.kq_hessian_accum(Xt, Ht, 1.0 / n, 0.0, ws)
    C = torch.empty((i, i), dtype=torch.float64, device=dev)
    K.kq_cross_accum(X, Xt, C, 1.0 / n, 0.0, ws)
    R0 = torch.empty((i, i), dtype=torch.float32, device=dev)
    info = torch.zeros(2, dtype=torch.int32, device=dev)
    K.kq_cholinv(Ht, sp.damp, R0, info[0:1], ws)
    Wstar = torch.empty((o, i), dtype=torch.float32, device=dev)
    K.kq_drift_target(W, C, R0, Wstar, ws)
    Sc = torch.empty((o, o) if cfg.form == "full" else HG.shape, dtype=torch.float32, device=dev)
    Sic = torch.empty_like(Sc)
    K.kq_hg_sqrt(HG, cfg.form, o, cfg.blk, Sc, Sic, info[1:2], ws)
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    out = {}
    for name, xa, xd in (("gptq_clean_H", X, None), ("gptq_drifted_H", Xt, None), ("drift_corrected", X, Xt)):
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            r = quantize_layer(xa, W, HG, s, t, cfg, ws=ws, S_cached=(Sc, Sic), verify=True, X_drift=xd)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        K.kq_kfac_loss(Wstar, r["What"], Ht, HG, cfg.form, cfg.blk, loss, ws)
        torch.cuda.synchronize()
        out[name] = {"layer_ms_S_cached": round(float(np.median(times)), 3), "drift_objective": float(loss.item())}
    ref = out["gptq_drifted_H"]["drift_objective"]
    for v in out.values():
        v["vs_gptq_drifted_H"] = round(v["drift_objective"] / ref, 5)
    return {"workload": sp.name, "drift_rel": rel, "variants": out}


def host_list(t) -> list:
    return [int(v) for v in t.cpu().tolist()]


def _blas_threads():
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limiter = None
    return cores, limiter


def _time_hessian_rotation(kq, HX, s_in, rows: int = 2048) -> tuple[float, str]:
    """Seconds of the oracle's H_X' = U^T H_X U: the row pass on at most `rows` rows of H_X, scaled to the
    i rows, times two (the column pass transforms i columns of the same length)."""
    i = HX.shape[0]
    r = min(rows, i)
    t0 = time.perf_counter()
    kq._rot(HX[:r], s_in, axis=1)
    dt = (time.perf_counter() - t0) * i / r * 2
    return dt, ("in full" if r == i else f"from {r} of {i} rows of one pass")


def _time_factor(kq, HX2, damp: float, cap: int = 4096) -> tuple[float, str]:
    """Seconds of the oracle's damped factor (inverse and Cholesky, O(i^3)): in full up to i = cap, else on
    the leading cap x cap block of the damped H, scaled by (i / cap)^3."""
    i = HX2.shape[0]
    k = min(i, cap)
    t0 = time.perf_counter()
    H, _ = kq.damped(HX2[:k, :k], damp)
    kq.inverse_upper_factor(H)
    dt = (time.perf_counter() - t0) * (i / k) ** 3
    return dt, ("in full" if k == i else f"on the leading {k} x {k} block scaled by (i/{k})^3")


def cpu_baseline(sp, full: bool = False) -> dict:
    """The float64 oracle, as it stands, on a bounded sample of the same layer (about 10-30 s of CPU work),
    timed per phase and scaled to the whole layer: H_X on at most 2048 tokens, the input rotation of W on
    at most 2048 rows (H_X's rotation in full), the output transform on at most 512 columns (all rows:
    it mixes rows), the sweep on at most 128 rows; the H_G square root and the damped factor in full.
    Stand-in values (rows of W'U, and an untimed factor of the unrotated H_X) feed the column-sampled output
    transform and the row-sampled sweep; the oracle's time does not depend on the values. Above 4096 the
    damped factor is timed on the leading 4096 x 4096 block and scaled by the cube of the width ratio, and
    the rotation of H_X on 2048 rows of one pass (scaled to both passes)."""
    from oracle import kronq as kq

    cores, limiter = _blas_threads()
    n_tok, r_in, c_out, n_rows = min(sp.n, 2048), min(sp.o, 2048), min(sp.i, 512), min(sp.o, 128)
    if full:
        n_tok, r_in, c_out, n_rows = sp.n, sp.o, sp.i, sp.o
    d = synth.layer_inputs(sp, x_rows=n_tok)
    X = synth.widen(d["X"], sp.x_dtype)
    W = synth.widen(d["W"], sp.w_dtype)
    HG = d["HG"].astype(np.float64)
    t = {}

    def done(phase: str) -> None:   # progress of the long full-size runs
        if full:
            print(f"# oracle {phase}: {t.get(phase, 0.0):.1f} s", file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    HX = kq.hessian(X)
    t["hessian"] = (time.perf_counter() - t0) * sp.n / n_tok
    done("hessian")
    del X
    t0 = time.perf_counter()
    W1 = kq.rotate_in_weights(W[:r_in], d["s"])
    t["rotate_in"] = (time.perf_counter() - t0) * sp.o / r_in
    if full:
        t0 = time.perf_counter()
        HX2 = kq.rotate_in_hessian(HX, d["s"])
        t["rotate_in"] += time.perf_counter() - t0
        done("rotate_in")
        how_rot = "in full"
    else:
        dt, how_rot = _time_hessian_rotation(kq, HX, d["s"])
        t["rotate_in"] += dt
    t0 = time.perf_counter()
    S, _ = kq.hg_sqrt(HG, sp.hg_form)
    t["hg_sqrt"] = time.perf_counter() - t0
    done("hg_sqrt")
    t0 = time.perf_counter()
    kq.rotate_out(W[:, :c_out], S, sp.hg_form, d["t"])
    t["rotate_out"] = (time.perf_counter() - t0) * sp.i / c_out
    done("rotate_out")
    if full:
        # the whole layer as the oracle computes it: R of the rotated H_X, the sweep on W'' = V S W'
        t0 = time.perf_counter()
        H, _ = kq.damped(HX2, sp.damp)
        R = kq.inverse_upper_factor(H)
        t["cholinv"] = time.perf_counter() - t0
        done("cholinv")
        how_fac = "in full"
        W2 = kq.rotate_out(W1, S, sp.hg_form, d["t"])
        print("# oracle: W'' for the sweep ready (untimed, the same product as rotate_out)", file=sys.stderr, flush=True)
    else:
        dt, how_fac = _time_factor(kq, HX, sp.damp)
        t["cholinv"] = dt
        # the sweep needs a factor of the whole width: R of the (unrotated) H_X, untimed, stands in for R of H_X'
        H, _ = kq.damped(HX, sp.damp)
        R = np.linalg.cholesky(np.linalg.inv(H)).T if sp.i <= 4096 else np.diag(1.0 / np.sqrt(np.diag(H)))
        W2 = W1
    if full:
        # rows are independent once R is fixed: the whole sweep in row chunks, with progress between them
        # (chunks of about a minute: the sweep's cost per row grows with the square of the width)
        t["quantize"] = 0.0
        chunk = 4096 if sp.i <= 4096 else 1024
        for r0 in range(0, sp.o, chunk):
            t0 = time.perf_counter()
            kq.sweep_blocked(W2[r0:r0 + chunk], R, sp.bits, sp.group, sp.block)
            t["quantize"] += time.perf_counter() - t0
            print(f"# oracle sweep: rows {r0}..{min(sp.o, r0 + chunk)} done ({t['quantize']:.0f} s)", file=sys.stderr,
                  flush=True)
    else:
        t0 = time.perf_counter()
        kq.sweep_blocked(W2[:n_rows], R, sp.bits, sp.group, sp.block)
        t["quantize"] = (time.perf_counter() - t0) * sp.o / n_rows
    done("quantize")
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    total = sum(t.values())
    if full:
        return {"value": sp.o * sp.i / total / 1e6, "unit": "Mweights/s", "cores": cores, "kind": "oracle",
                "sample": (f"float64 oracle on the whole layer, every phase in full (the sweep over row chunks of {chunk}, "
                           f"rows being independent once R is fixed); layer time {total:.1f} s"),
                "phases_s": {k: round(v, 3) for k, v in t.items()}}
    sample = (f"H_X on {n_tok} of {sp.n} tokens, rotation of W on {r_in} of {sp.o} rows, output transform on "
              f"{c_out} of {sp.i} columns, sweep on {n_rows} of {sp.o} rows (each scaled to the whole layer); "
              f"rotation of H_X {how_rot}, damped factor (of H_X: the same size and cost as of H_X') {how_fac}, "
              f"H_G square root (eigh) in full")
    return {"value": sp.o * sp.i / total / 1e6, "unit": "Mweights/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 oracle, {sample}; layer time {total:.1f} s",
            "phases_s": {k: round(v, 3) for k, v in t.items()}}


# ----------------------------------------------------------------------------- the 32-layer stack
def _stack_layer_host(li: int):
    """Host inputs of one layer of the stack (worker processes: numpy only)."""
    specs = synth.c5_specs(li)
    xs = {}
    for sp in specs:
        if sp.x_sub not in xs:
            xs[sp.x_sub] = (synth.gen_X(sp), synth.gen_signs(sp)[0])
    return xs, [(synth.gen_W(sp), synth.gen_HG(sp), synth.gen_signs(sp)[1], sp.x_sub) for sp in specs]


def stack_work() -> dict:
    """Algorithmic work of one pass over the stack, summed over its 224 sublayers and 128 inputs, with the
    per-layer formulas of algorithmic_work (H_X, its rotation and R once per distinct input)."""
    tot = {"hessian": 0, "rotate_in": 0, "rotate_out": 0, "cholinv": 0, "quantize": 0, "quantize_flop": 0}
    n = synth.C5_TOKENS
    for (_, o, i, x) in synth.C5_SUBLAYERS:
        tot["rotate_in"] += o * i * (2 + 4)
        tot["rotate_out"] += 8 * o * i
        tot["quantize"] += int((8 + 3 / 8 + 8 / 128) * o * i)   # at the 3.0-bit average
        tot["quantize_flop"] += o * i * (i - 128)
    for (_, i, _) in synth.C5_INPUTS:
        tot["hessian"] += n * i * (i + 1)
        tot["rotate_in"] += 32 * i * i
        tot["cholinv"] += 2 * i ** 3 // 3
        tot["quantize"] += 2 * i * i
    L = synth.C5_LAYERS
    return {"hessian": {"flop": L * tot["hessian"], "peak": "bf16_mfma"},
            "rotate_in": {"bytes": L * tot["rotate_in"], "peak": "hbm"},
            "rotate_out": {"bytes": L * tot["rotate_out"], "peak": "hbm"},
            "cholinv": {"flop": L * tot["cholinv"], "peak": "fp64_alu"},
            "quantize": {"bytes": L * tot["quantize"], "flop": L * tot["quantize_flop"], "peak": "hbm",
                         "flop_peak": "fp32_mfma"}}


def run_stack(steps: int, warmup: int):
    """The whole 32-layer stack: scores, allocation, then every sublayer quantized; `steps` timed passes
    after `warmup` passes over the first layer alone. Phase times from HIP events between the calls."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import torch

    from post_quantization_03_amd.stack import Layer, Sublayer, quantize_stack

    dev = torch.device("cuda:0")

    def to(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t0 = time.time()
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    layers = []
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("fork")) as ex:
        for li, (xs, subs) in enumerate(ex.map(_stack_layer_host, range(synth.C5_LAYERS))):
            layers.append(Layer(X=[to(xs[k][0], "bf16") for k in range(4)], s=[to(xs[k][1], "i8") for k in range(4)],
                                subs=[Sublayer(W=to(w, "bf16"), HG=to(h, "f32"), t=to(tt, "i8"), x=x)
                                      for (w, h, tt, x) in subs]))
            if li % 8 == 7:
                print(f"# stack inputs: {li + 1} layers on the device ({time.time() - t0:.0f}s)", file=sys.stderr,
                      flush=True)
    from post_quantization_03_amd.stack import _ws_bytes
    ws = torch.empty(_ws_bytes(layers, 128), dtype=torch.uint8, device=dev)
    for k in range(warmup):
        quantize_stack(layers[:1], ws=ws)
        torch.cuda.synchronize()
        print(f"# warmup {k + 1}/{warmup} done", file=sys.stderr, flush=True)
    times, phases = [], {}
    for k in range(steps):
        marks = []
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        out = quantize_stack(layers, ws=ws, marks=marks)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t_start)
        seq = [m for m in marks if len(m) == 2]
        for (name, a), (_, b) in zip(seq[:-1], seq[1:]):
            phases[name] = phases.get(name, 0.0) + a.elapsed_time(b) / steps
        for (name, a, b) in (m for m in marks if len(m) == 3):
            key = name + "_side"
            phases[key] = phases.get(key, 0.0) + a.elapsed_time(b) / steps
        print(f"# timed pass {k + 1}/{steps}: {times[-1]:.3f} s", file=sys.stderr, flush=True)
    if int(out.info.max().item()) != 0 or int(out.info.min().item()) != 0:
        raise RuntimeError("a factorisation failed in the stack")
    bits = np.array(out.bits)
    sizes = np.array([o * i for (_, o, i, _) in synth.C5_SUBLAYERS] * synth.C5_LAYERS)
    alloc = {"bits_2_3_4": np.bincount(bits, minlength=5)[2:].tolist(),
             "avg_bits": round(float(np.dot(bits, sizes) / sizes.sum()), 4)}
    return float(np.mean(times)) * 1e3, phases, alloc


def stack_cpu_baseline() -> dict:
    """The oracle on a bounded sample of the stack, scaled to all 32 layers: layer 0 with H_X on 1024 of
    8192 tokens per input, the rotation of H_X and the damped factor in full for its 4 inputs, and per
    sublayer the rotation of W on 512 rows, the output transform on 256 columns and the sweep on 64 rows
    (stand-in values), each scaled to the whole sublayer; then x32. The rotation of H_X and the damped
    factor are sampled as in cpu_baseline."""
    from oracle import kronq as kq

    cores, limiter = _blas_threads()
    n_tok, r_in, c_out, n_rows = 1024, 512, 256, 64
    specs = synth.c5_specs(0)
    t = {"hessian": 0.0, "rotate_in": 0.0, "hg_sqrt": 0.0, "rotate_out": 0.0, "cholinv": 0.0, "quantize": 0.0}
    Rs, ss = {}, {}
    for sp in specs:
        if sp.x_sub in Rs:
            continue
        X = synth.widen(synth.gen_X(sp, n_tok), "bf16")
        s_in = synth.gen_signs(sp)[0]
        t0 = time.perf_counter()
        HX = kq.hessian(X)
        t["hessian"] += (time.perf_counter() - t0) * sp.n / n_tok
        dt, _ = _time_hessian_rotation(kq, HX, s_in)
        t["rotate_in"] += dt
        dt, _ = _time_factor(kq, HX, 0.01)
        t["cholinv"] += dt
        H, _ = kq.damped(HX, 0.01)
        # untimed stand-in factor of the whole width for the sampled sweeps
        Rs[sp.x_sub] = np.diag(1.0 / np.sqrt(np.diag(H)))
        ss[sp.x_sub] = s_in
    for sp in specs:
        W = synth.widen(synth.gen_W(sp), "bf16")
        h = synth.gen_HG(sp).astype(np.float64)
        tt = synth.gen_signs(sp)[1]
        t0 = time.perf_counter()
        W1 = kq.rotate_in_weights(W[:r_in], ss[sp.x_sub])
        t["rotate_in"] += (time.perf_counter() - t0) * sp.o / r_in
        t0 = time.perf_counter()
        S, _ = kq.hg_sqrt(h, "diag")
        t["hg_sqrt"] += time.perf_counter() - t0
        t0 = time.perf_counter()
        kq.rotate_out(W[:, :c_out], S, "diag", tt)
        t["rotate_out"] += (time.perf_counter() - t0) * sp.i / c_out
        t0 = time.perf_counter()
        kq.sweep_blocked(W1[:n_rows], Rs[sp.x_sub], 3, 128, 128)
        t["quantize"] += (time.perf_counter() - t0) * sp.o / n_rows
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    layer = sum(t.values())
    total = layer * synth.C5_LAYERS
    weights = sum(o * i for (_, o, i, _) in synth.C5_SUBLAYERS) * synth.C5_LAYERS
    return {"value": weights / total / 1e6, "unit": "Mweights/s", "cores": cores, "kind": "oracle",
            "sample": (f"float64 oracle on layer 0 of 32 (extrapolated x32): H_X on {n_tok} of 8192 tokens per input, "
                       f"rotation of H_X from 2048 rows of one pass, damped factor on at most a 4096 x 4096 block "
                       f"(scaled by the cube of the width ratio), per sublayer the rotation of W on {r_in} rows, "
                       f"the output transform on {c_out} columns and the sweep on {n_rows} rows, each scaled; "
                       f"stack time {total:.0f} s"),
            "phases_s": {k: round(v * synth.C5_LAYERS, 2) for k, v in t.items()}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="C2", choices=["C1", "C2", "C3", "C4", "C5"],
                    help="C2 (default) is the 4096 x 4096 layer the metric is quoted on; C1, C3, C4 the other layers; "
                         "C5 the 32-layer stack (one timed pass by default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phases", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (fp32 elementwise kernel), the reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    ap.add_argument("--hg-variants", action="store_true",
                    help="quantize the C2 layer with H_G prepared in several ways (exact, 128-block, diagonal, "
                         "low-rank of several ranks, none) and print the exact K-FAC loss of each as its own JSON line")
    ap.add_argument("--solver-variants", action="store_true",
                    help="run the workload's layer with the Hessian-aware grid search and/or trace-ordered blocks and "
                         "print time and exact K-FAC loss of each as its own JSON line")
    ap.add_argument("--drift", action="store_true",
                    help="compare GPTQ with the input-drift-corrected solver on drifted synthetic inputs and print "
                         "the result as its own JSON line")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the float64 oracle on the whole workload layer (every phase in full, minutes for the "
                         "large layers) and print it as a JSON line (no GPU work)")
    ap.add_argument("--probe-peaks", action="store_true",
                    help="measure the fp64/fp32 vector and fp64/fp32/bf16 matrix-core throughput and the HBM copy rate "
                         "of this GPU (prints a JSON line, not the benchmark line)")
    ap.add_argument("--profile-phases", action="store_true",
                    help="for rocprofv3 counter runs: each phase of the workload's layer alone, twice, after one full "
                         "step, with a marker dispatch before each (prints a JSON line naming the phases, not the "
                         "benchmark line)")
    ap.add_argument("--matvec-only", action="store_true",
                    help="time only the inference-side product (kq_matvec_quantized) on the workload's layer shape "
                         "with random codes, and print its own JSON line (not the benchmark line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the per-layer solver runs on a single MI355X in this build "
              "(multi-GPU sharding is described in DESIGN.md, not implemented).", file=sys.stderr)
        sys.exit(2)
    if args.probe_peaks:
        print(json.dumps({"probe_peaks": probe_peaks()}), flush=True)
        return
    if args.workload == "C5":
        run_stack_line(args)
        return
    sp = synth.CONFIGS[args.workload]
    if args.cpu_full:
        print(json.dumps({"workload": sp.name, "cpu_oracle_full": cpu_baseline(sp, full=True)}), flush=True)
        return
    if args.profile_phases:
        profile_phases(sp)
        return
    if args.drift:
        print(json.dumps(drift_study(sp)), flush=True)
        return
    if args.solver_variants:
        print(json.dumps(solver_variants(sp)), flush=True)
        return
    if args.hg_variants:
        print(json.dumps(hg_variants(sp)), flush=True)
        return
    if args.matvec_only:
        print(json.dumps({"workload": sp.name, "o": sp.o, "i": sp.i, "bits": sp.bits, "group": sp.group,
                          "hg_form": sp.hg_form, "matvec_quantized": matvec_only(sp)}), flush=True)
        return
    if args.copy_calibration:
        import torch
        src = torch.ones(args.copy_calibration * (1 << 18), dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(f"# copy calibration: read {src.numel() * 4} B, wrote {dst.numel() * 4} B", file=sys.stderr, flush=True)
        del src, dst
    ms, ph, out, iters, mv, ms_cached = run_gpu(sp, args.steps, args.warmup, not args.no_phases)
    value = sp.o * sp.i / (ms / 1e3) / 1e6
    roof, per_phase, s_cached, aggregates, chain = None, None, None, None, None
    if ph:
        chain_ms = ph.pop("_chain")
        chain = {"rows": 16, "ms": round(chain_ms, 4), "per_step_ns": round(chain_ms / sp.i * 1e6, 2),
                 "quantize_ms": round(ph["quantize"], 4), "quantize_over_chain": round(ph["quantize"] / chain_ms, 3)}
        work = algorithmic_work(sp, iters)
        per_phase = {k: roofline_of(k, work[k], ph[k]) for k in work if k in ph and
                     (work[k].get("flop") or work[k].get("bytes"))}
        dom = max(per_phase, key=lambda k: ph[k])
        roof = per_phase[dom]
        roof["traffic"] = measured_traffic(dom) if sp.name.startswith("C2") else None
        if ms_cached:
            s_cached = round(sp.o * sp.i / (ms_cached / 1e3) / 1e6, 3)
        # aggregates over the phases, each phase taken at its own bound: FLOP-weighted for the dense
        # contractions (algorithmic FLOP / sum of time x peak), byte-weighted for the HBM-bound ones
        dense = [k for k in per_phase if per_phase[k]["unit"] == "TFLOP/s"]
        hbm = [k for k in per_phase if per_phase[k]["unit"] == "GB/s"]
        aggregates = {
            "dense_phases": dense,
            "dense_frac": round(sum(work[k]["flop"] for k in dense) /
                                sum(ph[k] / 1e3 * per_phase[k]["peak"] * 1e12 for k in dense), 4) if dense else None,
            "hbm_phases": hbm,
            "hbm_frac": round(sum(work[k]["bytes"] for k in hbm) / (sum(ph[k] for k in hbm) / 1e3 * PEAK["hbm"]), 4)
            if hbm else None,
        }
    cpu = None if args.no_cpu_baseline else cpu_baseline(sp)
    line = {"metric": "layer-quant throughput: Mweights/s (4096x4096 W3 g128) + % MFMA/HBM peak",
            "value": round(value, 3), "unit": "Mweights/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
            "config": {"workload": sp.name, "o": sp.o, "i": sp.i, "tokens": sp.n, "x_dtype": sp.x_dtype,
                       "hg_form": sp.hg_form, "bits": sp.bits, "group": sp.group,
                       "arith": "bf16 MFMA (exact products, fp64 accumulation) for H_X; fp64 for H_G^1/2 "
                                "and the damped factor; fp32 for the rotations of W and the sweep"},
            "phases_ms": {k: round(v, 4) for k, v in ph.items()} if ph else None,
            "db_steps": iters[0], "db_last_step": ("newton-schulz" if iters[1] else "denman-beavers")
            if iters[0] else None, "s_cached_mweights_per_s": s_cached,
            "roofline": roof, "phases_roofline": per_phase, "phases_aggregate": aggregates,
            "sweep_critical_path": chain, "cpu_baseline": cpu, "matvec_quantized": mv}
    print(json.dumps(line), flush=True)


def probe_peaks() -> dict:
    """Measured ceilings of the execution units and HBM on this GPU (libkqprobe.so): dependency-free
    fp64/fp32 vector FMA loops, fp64/fp32/bf16 matrix-core loops over every compute unit, and a 4 GiB
    device copy; each timed with HIP events after a warm-up launch. The vendor figures (PEAK) stay the
    roofline denominators; these say what the units deliver here."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "post_quantization_03_amd", "libkqprobe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m post_quantization_03_amd.build`")
    L = ctypes.CDLL(path)
    L.kq_probe_run.restype = ctypes.c_int
    L.kq_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    dev = torch.device("cuda:0")
    scratch = torch.empty(8 << 20, dtype=torch.uint8, device=dev)
    nbytes = 4 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    kinds = {"fp64_vector_fma": (0, 20000, "TFLOP/s", 78.6), "fp64_mfma_16x16x4": (1, 20000, "TFLOP/s", 78.6),
             "fp32_mfma_16x16x4": (2, 20000, "TFLOP/s", 157.3), "bf16_mfma_16x16x32": (3, 20000, "TFLOP/s", 2500.0),
             "fp32_vector_fma": (4, 20000, "TFLOP/s", 157.3), "hbm_copy": (5, 0, "GB/s", 8000.0),
             "fp64_mfma_and_vector_side_by_side": (6, 20000, "TFLOP/s", 78.6)}
    out = {}
    for name, (kind, iters, unit, vendor) in kinds.items():
        sec, work = ctypes.c_double(), ctypes.c_double()
        rc = L.kq_probe_run(kind, iters, nbytes, scratch.data_ptr(), src.data_ptr(), dst.data_ptr(),
                            ctypes.byref(sec), ctypes.byref(work))
        if rc != 0:
            raise RuntimeError(f"probe {name} failed ({rc})")
        rate = work.value / sec.value / (1e12 if unit == "TFLOP/s" else 1e9)
        out[name] = {"measured": round(rate, 2), "unit": unit, "vendor_peak": vendor, "frac_of_vendor": round(rate / vendor, 3),
                     "ms": round(sec.value * 1e3, 3)}
        print(f"# probe {name}: {rate:.1f} {unit}", file=sys.stderr, flush=True)
    return out


PROFILE_PHASES = ("copy", "hessian", "rotate_in", "hg_sqrt", "rotate_out", "cholinv", "quantize")


def profile_phases(sp, reps: int = 2) -> None:
    """For counter collection: one full layer step (which leaves every intermediate in place), then a plain
    fp32 copy of 64 MiB (the reference that scales FETCH_SIZE / WRITE_SIZE to bytes), then each phase of
    the layer alone, `reps` times. A marker dispatch (kq_hg_extract on a 4 x 4 matrix: hg_extract_kernel,
    which the layer never runs) precedes the copy and every phase, so that the profiler's per-dispatch
    records split into PROFILE_PHASES in that order."""
    import torch

    from post_quantization_03_amd import _lib as K
    from post_quantization_03_amd.layer import LayerCfg, hg_factor_shape, quantize_layer, workspace_bytes

    dev = torch.device("cuda:0")
    d = synth.layer_inputs(sp)

    def to(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    X, W, HG = to(d["X"], sp.x_dtype), to(d["W"], sp.w_dtype), to(d["HG"], "f32")
    s, t = to(d["s"], "i8"), to(d["t"], "i8")
    del d
    cfg = LayerCfg(bits=sp.bits, group=sp.group, damp=sp.damp, form=sp.hg_form,
                   blk=sp.hg_blk if sp.hg_form == "block" else 0)
    xdt = K.KQ_BF16 if sp.x_dtype == "bf16" else K.KQ_F32
    ws = torch.empty(workspace_bytes(sp.o, sp.i, sp.n, xdt, cfg), dtype=torch.uint8, device=dev)
    quantize_layer(X, W, HG, s, t, cfg, ws=ws)
    torch.cuda.synchronize()
    o, i, n = sp.o, sp.i, sp.n
    f32 = dict(dtype=torch.float32, device=dev)
    H = torch.empty((i, i), dtype=torch.float64, device=dev)
    W2 = torch.empty((o, i), **f32)
    S = torch.empty(hg_factor_shape(o, cfg), **f32)
    R = torch.empty((i, i), **f32)
    info = torch.zeros(2, dtype=torch.int32, device=dev)
    ng = i // cfg.group if cfg.group else 1
    codes = torch.empty((o, i * cfg.bits // 32), dtype=torch.int32, device=dev)
    scale, offset, rl = torch.empty((o, ng), **f32), torch.empty((o, ng), **f32), torch.empty((o,), **f32)
    Hm, hm = torch.eye(4, dtype=torch.float64, device=dev), torch.empty(4, **f32)
    src = torch.ones(64 << 18, **f32)
    dst = torch.empty_like(src)
    calls = {
        "copy": lambda: torch.mul(src, 1.0, out=dst),
        "hessian": lambda: K.kq_hessian_accum(X, H, 1.0 / n, 0.0, ws),
        "rotate_in": lambda: K.kq_rotate_in(W, W2, H, s, ws),
        "hg_sqrt": lambda: K.kq_hg_sqrt(HG, cfg.form, o, cfg.blk, S, None, info[0:1], ws),
        "rotate_out": lambda: K.kq_rotate_out(W2, S, cfg.form, cfg.blk, t, ws),
        "cholinv": lambda: K.kq_cholinv(H, cfg.damp, R, info[1:2], ws),
        "quantize": lambda: K.kq_quantize_layer(W2, R, cfg.bits, cfg.group, cfg.block, codes, scale, offset, rl, ws),
    }
    for name in PROFILE_PHASES:
        K.kq_hg_extract(Hm, "diag", 0, hm)
        for _ in range(1 if name == "copy" else reps):
            calls[name]()
        torch.cuda.synchronize()
        print(f"# profiled phase {name}", file=sys.stderr, flush=True)
    print(json.dumps({"profiled": sp.name, "phases": PROFILE_PHASES, "reps": reps, "copy_bytes": src.numel() * 4}),
          flush=True)


def run_stack_line(args) -> None:
    """One JSON line for the 32-layer stack (C5): whole-stack throughput, summed phase times, the
    allocation, per-phase roofline and the oracle on a bounded sample."""
    steps = args.steps if args.steps != 5 else 1   # one pass by default: a pass quantizes 6.5e9 weights
    ms, ph, alloc = run_stack(steps, args.warmup if args.warmup != 2 else 1)
    weights = sum(o * i for (_, o, i, _) in synth.C5_SUBLAYERS) * synth.C5_LAYERS
    work = stack_work()
    # the damped factors (and the rotations of H_X before them) run on their own streams, beside the
    # sublayers' work: their phase times are the sums of their own intervals, which overlap the rest
    ph_work = dict(ph)
    ph_work["cholinv"] = ph.get("cholinv_side", 0.0)
    ph_work["rotate_in"] = ph.get("rotate_in", 0.0) + ph.get("rotate_in_side", 0.0)
    per_phase = {k: roofline_of(k, work[k], ph_work[k]) for k in work if ph_work.get(k)}
    dense = [k for k in per_phase if per_phase[k]["unit"] == "TFLOP/s"]
    hbm = [k for k in per_phase if per_phase[k]["unit"] == "GB/s"]
    aggregates = {
        "dense_phases": dense,
        "dense_frac": round(sum(work[k]["flop"] for k in dense) /
                            sum(ph_work[k] / 1e3 * per_phase[k]["peak"] * 1e12 for k in dense), 4),
        "hbm_phases": hbm,
        "hbm_frac": round(sum(work[k]["bytes"] for k in hbm) / (sum(ph_work[k] for k in hbm) / 1e3 * PEAK["hbm"]), 4),
    }
    dom = max(per_phase, key=lambda k: ph_work[k])
    cpu = None if args.no_cpu_baseline else stack_cpu_baseline()
    line = {"metric": "layer-quant throughput: Mweights/s (4096x4096 W3 g128) + % MFMA/HBM peak",
            "value": round(weights / (ms / 1e3) / 1e6, 3), "unit": "Mweights/s", "n_gpus": 1, "steps": steps,
            "warmup": args.warmup if args.warmup != 2 else 1, "ms_per_step": round(ms, 2), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
            "config": {"workload": "C5 32-layer stack x 7 sublayers, {2,3,4} bits under a 3.0 budget, g128",
                       "layers": synth.C5_LAYERS, "tokens": synth.C5_TOKENS, "weights": weights, "hg_form": "diag",
                       "allocation": alloc},
            "phases_ms": {k: round(v, 3) for k, v in ph.items()},
            "roofline": per_phase[dom], "phases_roofline": per_phase, "phases_aggregate": aggregates,
            "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
