"""Mixed-precision quantization of a stack of layers through the C ABI (include/kq.h).

KronQ review page, Method (2) and Comparison: every sublayer is scored with tr(H_G) tr(H_X), the
scores order sublayer bit upgrades under an average budget, then every sublayer is quantized with the
unchanged per-layer solver.

Pass 1 (per layer): H_X for each distinct input (kq_hessian_accum), the score of every sublayer that
reads it (kq_sensitivity). Host: kq_allocate_bits over all scores.
Pass 2 (per layer): per distinct input one rotation of H_X and one damped factor R (kq_rotate_in with
no weights, kq_cholinv): sublayers that read the same input share U and R. Per sublayer: kq_rotate_in
(weights), kq_hg_sqrt, kq_rotate_out, kq_quantize_layer at its bit-width.

The damped factors depend only on pass 1, and each one is a chain of small dependent steps, so they run
on streams of their own (one per distinct input of a layer, each with its own workspace), ahead of and
beside the sublayers' work on the caller's stream, which waits only for the factor it needs.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import _lib as K


@dataclass
class Sublayer:
    W: torch.Tensor          # o x i, bf16 or fp32
    HG: torch.Tensor         # diagonal H_G (o)
    t: torch.Tensor          # output-side signs (o)
    x: int                   # index of the input it reads


@dataclass
class Layer:
    X: list                  # calibration activations per distinct input (n x i)
    s: list                  # input-side signs per distinct input
    subs: list               # Sublayer


@dataclass
class StackOut:
    scores: torch.Tensor
    bits: list
    codes: list = field(default_factory=list)
    scale: list = field(default_factory=list)
    offset: list = field(default_factory=list)
    row_loss: list = field(default_factory=list)
    Q: list = field(default_factory=list)
    R: list = field(default_factory=list)
    H: list = field(default_factory=list)


_FACTOR_STREAMS: dict = {}


def _factor_streams(dev, count: int) -> list:
    """Streams (default priority) for the damped factors, kept per device."""
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    have = _FACTOR_STREAMS.setdefault(key, [])
    while len(have) < count:
        have.append(torch.cuda.Stream(device=dev))
    return have[:count]


def _factor_ws_bytes(layers) -> int:
    need = 256
    for L in layers:
        for X in L.X:
            i = X.shape[1]
            need = max(need, K.kq_workspace_bytes("rotate_in", 0, i), K.kq_workspace_bytes("cholinv", 0, i))
    return need


def _ws_bytes(layers, group: int) -> int:
    need = 256
    for L in layers:
        for x, X in enumerate(L.X):
            n, i = X.shape
            need = max(need, K.kq_workspace_bytes("hessian", 0, i, n), K.kq_workspace_bytes("rotate_in", 0, i),
                       K.kq_workspace_bytes("cholinv", 0, i))
        for sl in L.subs:
            o, i = sl.W.shape
            need = max(need, K.kq_workspace_bytes("rotate_in", o, i), K.kq_workspace_bytes("rotate_out", o, i),
                       K.kq_workspace_bytes("quantize", o, i))
    return need


def quantize_stack(layers: list, budget: float = 3.0, group: int = 128, damp: float = 0.01, keep_q: bool = False,
                   keep_h: bool = False, ws: torch.Tensor | None = None, H_cache: list | None = None,
                   marks: list | None = None) -> StackOut:
    """``marks``: when a list is given, a timing event is recorded on the current stream before every
    call, as (phase name, event), and one ("end", event) after the last; the time from one mark to the
    next belongs to the first one's phase. Work on the factor streams is marked by its own start and
    end events, as (phase name, start, end); those intervals overlap the caller's stream's."""
    dev = layers[0].X[0].device

    def mark(name: str) -> None:
        if marks is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.append((name, e))

    if ws is None:
        ws = torch.empty(_ws_bytes(layers, group), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    nsub = sum(len(L.subs) for L in layers)
    scores = torch.empty(nsub, dtype=torch.float64, device=dev)
    # ---- pass 1: H_X per distinct input, scores
    Hs = []
    k = 0
    for li, L in enumerate(layers):
        hl = []
        for x, X in enumerate(L.X):
            n, i = X.shape
            H = H_cache[li][x] if H_cache is not None else torch.empty((i, i), dtype=torch.float64, device=dev)
            mark("hessian")
            K.kq_hessian_accum(X, H, 1.0 / n, 0.0, ws)
            hl.append(H)
        for sl in L.subs:
            o = sl.W.shape[0]
            mark("sensitivity")
            K.kq_sensitivity(hl[sl.x], sl.HG, "diag", o, 0, scores[k:k + 1])
            k += 1
        Hs.append(hl)
    sizes = [sl.W.shape[0] * sl.W.shape[1] for L in layers for sl in L.subs]
    mark("allocate")
    bits = K.kq_allocate_bits(scores.cpu().numpy(), sizes, budget, 2, 4).tolist()
    out = StackOut(scores=scores, bits=bits)
    # ---- pass 2
    # info[layer, input] from the damped factors, info[layer, 8 + sublayer] from the H_G roots
    info = torch.zeros((len(layers), 16), dtype=torch.int32, device=dev)
    main = torch.cuda.current_stream(dev)
    nf = max(len(L.X) for L in layers)
    fstreams = _factor_streams(dev, nf)
    fbytes = _factor_ws_bytes(layers)
    fws = []
    for fs in fstreams:
        fs.wait_stream(main)   # pass 1 (H_X) and the allocations above
        with torch.cuda.stream(fs):
            fws.append(torch.empty(fbytes, dtype=torch.uint8, device=dev))
    mark("factors_enqueued")
    k = 0
    for li, L in enumerate(layers):
        Rs, ready = [], []
        for x, H in enumerate(Hs[li]):
            i = H.shape[0]
            fs = fstreams[x]
            with torch.cuda.stream(fs):
                t = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if marks is not None else None
                if t:
                    t[0].record(fs)
                K.kq_rotate_in_hessian(H, L.s[x], fws[x])
                R = torch.empty((i, i), **f32)
                if t:
                    t[1].record(fs)
                K.kq_cholinv(H, damp, R, info[li, x:x + 1], fws[x])
                ev = torch.cuda.Event(enable_timing=t is not None)
                ev.record(fs)
                if t:
                    marks.append(("rotate_in", t[0], t[1]))
                    marks.append(("cholinv", t[1], ev))
            R.record_stream(main)
            H.record_stream(fs)
            Rs.append(R)
            ready.append(ev)
        for j, sl in enumerate(L.subs):
            o, i = sl.W.shape
            b = bits[k]
            mark("wait_factor")
            main.wait_event(ready[sl.x])
            W2 = torch.empty((o, i), **f32)
            mark("rotate_in")
            K.kq_rotate_in(sl.W, W2, None, L.s[sl.x], ws)
            S = torch.empty((o,), **f32)
            mark("hg_sqrt")
            K.kq_hg_sqrt(sl.HG, "diag", o, 0, S, None, info[li, 8 + j:9 + j], ws)
            mark("rotate_out")
            K.kq_rotate_out(W2, S, "diag", 0, sl.t, ws)
            ng = i // group if group else 1
            codes = torch.empty((o, i * b // 32), dtype=torch.int32, device=dev)
            scale = torch.empty((o, ng), **f32)
            offset = torch.empty((o, ng), **f32)
            rl = torch.empty((o,), **f32)
            mark("quantize")
            K.kq_quantize_layer(W2, Rs[sl.x], b, group, 128, codes, scale, offset, rl, ws)
            out.codes.append(codes)
            out.scale.append(scale)
            out.offset.append(offset)
            out.row_loss.append(rl)
            if keep_q:
                out.Q.append(W2)
            k += 1
        if keep_h:
            out.H.append(Hs[li])
            out.R.append(Rs)
    for fs in fstreams:
        main.wait_stream(fs)
    out.info = info
    mark("end")
    return out

