"""One-layer KronQ pipeline on the GPU through the C ABI (include/kq.h).

Order of the calls (KronQ review page, Method and Key idea):
  kq_hessian_accum  H_X = X^T X / n
  kq_sensitivity    tr(H_G) tr(H_X)         (before the rotation: undamped, unrotated H_X)
  kq_rotate_in      W' = W U, H_X' = U^T H_X U
  kq_cholinv        R with (H_X' + lambda I)^{-1} = R^T R
  kq_hg_sqrt        S = H_G^{1/2}, S^{-1}    (skipped when a cached S is passed; for block and full H_G
                                             on a second stream forked before the four calls above,
                                             which do not depend on it, and run concurrently with them)
  kq_rotate_out     W'' = V S W'
  kq_quantize_layer GPTQ sweep on W'' -> codes, scale, offset, w^ (rotated), row loss
Torch only allocates device memory and supplies the streams.

The returned info (device int32 [2]) must be read by the caller once the stream is synchronised:
info[0] from kq_hg_sqrt, info[1] from kq_cholinv, 0 on success. info[0] = -1 means a device-side
wait of the square root's sweep ran out after its first step (the device stopped running the sweep's
two queues side by side): S, and so every output, is invalid and the layer should be run again.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import torch

from . import _lib as K


@dataclass
class LayerCfg:
    bits: int
    group: int = 128
    block: int = 128
    damp: float = 0.01
    form: str = "diag"      # H_G storage form
    blk: int = 0            # block size of a block-diagonal H_G
    search: int = 0         # candidates of the Hessian-aware grid search (0: min-max grids)
    order: str = "natural"  # "natural" or "trace": 128-column blocks in descending trace of H_X'


_SIDE: dict = {}
_WORKER: dict = {}


def _sqrt_worker(dev) -> ThreadPoolExecutor:
    """One host thread per device, kept for the process, that enqueues the square root (its one readback
    uses a pinned buffer of the calling thread, allocated once)."""
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key not in _WORKER:
        _WORKER[key] = ThreadPoolExecutor(max_workers=1, thread_name_prefix=f"kq_hg_sqrt{key}")
    return _WORKER[key]


def _side_stream(dev):
    """One second stream per device (default priority) for the H_G square root."""
    import torch
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key not in _SIDE:
        _SIDE[key] = torch.cuda.Stream(device=dev)
    return _SIDE[key]


def workspace_bytes(o: int, i: int, n: int, xdt: int, cfg: LayerCfg, verify: bool = False) -> int:
    ops = ["hessian", "rotate_in", "hg_sqrt", "rotate_out", "cholinv", "quantize"] + (["unrotate", "loss"] if verify else [])
    return max(K.kq_workspace_bytes(op, o, i, n, xdt, cfg.bits, cfg.group, cfg.form, cfg.blk) for op in ops)


def hg_factor_shape(o: int, cfg: LayerCfg):
    if cfg.form == "diag":
        return (o,)
    if cfg.form == "block":
        return (o // cfg.blk, cfg.blk, cfg.blk)
    return (o, o)


def quantize_layer(X: torch.Tensor, W: torch.Tensor, HG: torch.Tensor, s: torch.Tensor, t: torch.Tensor,
                   cfg: LayerCfg, ws: torch.Tensor | None = None, S_cached=None, verify: bool = False,
                   x_batch: int | None = None, X_drift: torch.Tensor | None = None) -> dict:
    """All steps of the per-layer solver on device-resident inputs. Returns device tensors.
    X_drift: the layer's inputs once earlier layers are quantized; the sweep then runs on the drift
    target W* = W C (H~ + lambda I)^{-1} with H~ from X_drift (kq_drift_target)."""
    dev = W.device
    o, i = W.shape
    n = X.shape[0]
    xdt = K.KQ_BF16 if X.dtype == torch.bfloat16 else K.KQ_F32
    if ws is None:
        ws = torch.empty(max(workspace_bytes(o, i, n if x_batch is None else min(n, x_batch), xdt, cfg, verify), 256),
                         dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    info = torch.zeros((2,), dtype=torch.int32, device=dev)
    join = None
    if S_cached is None:
        S = torch.empty(hg_factor_shape(o, cfg), **f32)
        Sinv = torch.empty_like(S) if verify else None
        if cfg.form != "diag":
            # S depends on H_G alone: it runs on the second stream, forked here (after the inputs and
            # outputs above exist) and joined before kq_rotate_out. kq_hg_sqrt returns only once its
            # first step has run on the device, and enqueueing the H_X chain can block the host too
            # (the damped factor's ~150 launches fill the stream's hardware queue, so the host waits
            # for the device to work through them), so the square root is enqueued from a host thread
            # of its own, started here: both chains reach the device at once.
            join = _side_stream(dev)
            join.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(join):
                ws_s = torch.empty(max(K.kq_workspace_bytes("hg_sqrt", o, 0, form=cfg.form, blk=cfg.blk), 256),
                                   dtype=torch.uint8, device=dev)

            def _sqrt():
                torch.cuda.set_device(dev)
                K.kq_hg_sqrt(HG, cfg.form, o, cfg.blk, S, Sinv, info[0:1], ws_s, stream=join)

            sqrt_done = _sqrt_worker(dev).submit(_sqrt)
    else:
        S, Sinv = S_cached
    H = torch.empty((i, i), dtype=torch.float64, device=dev)
    Xh = X if X_drift is None else X_drift
    if x_batch is None or x_batch >= n:
        K.kq_hessian_accum(Xh, H, 1.0 / n, 0.0, ws)
    else:
        for k0 in range(0, n, x_batch):
            K.kq_hessian_accum(Xh[k0:k0 + x_batch], H, 1.0 / n, 0.0 if k0 == 0 else 1.0, ws)
    if X_drift is not None:
        C = torch.empty((i, i), dtype=torch.float64, device=dev)
        wsx = torch.empty(max(K.kq_workspace_bytes("cross", 0, i, n), K.kq_workspace_bytes("drift", o, i),
                              K.kq_workspace_bytes("cholinv", o, i)), dtype=torch.uint8, device=dev)
        K.kq_cross_accum(X, X_drift, C, 1.0 / n, 0.0, wsx)
        R0 = torch.empty((i, i), **f32)
        info0 = torch.zeros((1,), dtype=torch.int32, device=dev)
        K.kq_cholinv(H, cfg.damp, R0, info0, wsx)
        Wt = torch.empty((o, i), **f32)
        K.kq_drift_target(W, C, R0, Wt, wsx)
        del C, R0, wsx
        W = Wt
    score = torch.empty((1,), dtype=torch.float64, device=dev)
    K.kq_sensitivity(H, HG, cfg.form, o, cfg.blk, score)
    W2 = torch.empty((o, i), **f32)
    K.kq_rotate_in(W, W2, H, s, ws)
    R = torch.empty((i, i), **f32)
    if cfg.order != "trace":
        K.kq_cholinv(H, cfg.damp, R, info[1:2], ws)
    if join is not None:
        sqrt_done.result()   # the square root is enqueued (its errors are raised here)
        for t_ in (S, Sinv, info, HG, ws_s):
            if t_ is not None:
                t_.record_stream(join)
        torch.cuda.current_stream(dev).wait_stream(join)
    elif S_cached is None:
        K.kq_hg_sqrt(HG, cfg.form, o, cfg.blk, S, Sinv, info[0:1], ws)
    K.kq_rotate_out(W2, S, cfg.form, cfg.blk, t, ws)
    W2_in = W2.clone() if verify else None
    ng = i // cfg.group if cfg.group else 1
    codes = torch.empty((o, i * cfg.bits // 32), dtype=torch.int32, device=dev)
    scale = torch.empty((o, ng), **f32)
    offset = torch.empty((o, ng), **f32)
    row_loss = torch.empty((o,), **f32)
    order = None
    if cfg.order == "trace":
        # blocks in descending trace of H_X': permute W'' and H_X' forward, factor and sweep there,
        # then move the outputs back (groups and packed words stay inside 128-column blocks)
        nb = i // cfg.block
        order = torch.empty((2 * nb,), dtype=torch.int32, device=dev)
        K.kq_block_order(H, cfg.block, order)
        Ht, Hp = torch.empty_like(H), torch.empty_like(H)
        K.kq_permute_blocks(H, Ht, cfg.block, 0, order[:nb])
        K.kq_permute_blocks(Ht, Hp, cfg.block, 1, order[:nb])
        del Ht
        Wp = torch.empty_like(W2)
        K.kq_permute_blocks(W2, Wp, cfg.block, 0, order[:nb])
        K.kq_cholinv(Hp, cfg.damp, R, info[1:2], ws)
        del Hp
        cp = torch.empty_like(codes)
        # per-row grids (group 0) do not move; group grids move with their blocks
        sp_, op_ = (torch.empty_like(scale), torch.empty_like(offset)) if cfg.group else (scale, offset)
        K.kq_quantize_layer_search(Wp, R, cfg.bits, cfg.group, cfg.block, cfg.search, cp, sp_, op_, row_loss, ws)
        back = order[nb:]
        K.kq_permute_blocks(Wp, W2, cfg.block, 0, back)
        K.kq_permute_blocks(cp, codes, cfg.block * cfg.bits // 32, 0, back)
        if cfg.group:
            K.kq_permute_blocks(sp_, scale, cfg.block // cfg.group, 0, back)
            K.kq_permute_blocks(op_, offset, cfg.block // cfg.group, 0, back)
    else:
        K.kq_quantize_layer_search(W2, R, cfg.bits, cfg.group, cfg.block, cfg.search, codes, scale, offset, row_loss,
                                   ws)
    out = {"H": H, "score": score, "Q": W2, "R": R, "codes": codes, "scale": scale, "offset": offset,
           "row_loss": row_loss, "info": info, "S": S, "Sinv": Sinv, "order": order}
    if verify:
        What = torch.empty((o, i), **f32)
        K.kq_unrotate(W2, s, t, Sinv, cfg.form, cfg.blk, What, ws)
        loss = torch.empty((1,), dtype=torch.float64, device=dev)
        loss_rows = torch.empty((o,), dtype=torch.float64, device=dev)
        K.kq_layer_loss(W2_in, W2, H, loss_rows, loss, ws)
        out.update({"W2": W2_in, "What": What, "loss": loss, "loss_rows": loss_rows})
    return out
