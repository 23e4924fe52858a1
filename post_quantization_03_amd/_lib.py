"""ctypes binding of libkq.so (include/kq.h). Argument marshalling only: every step runs in the
library's HIP kernels. Tensors supply device pointers; the stream is torch's current stream.

The library must be built (python -m post_quantization_03_amd.build); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkq.so")

KQ_F32, KQ_BF16 = 0, 1
HG_FORM = {"diag": 0, "block": 1, "full": 2}
OP = {"hessian": 0, "rotate_in": 1, "hg_sqrt": 2, "rotate_out": 3, "cholinv": 4, "quantize": 5, "unrotate": 6,
      "loss": 7, "matvec": 8, "hg_lowrank": 9, "kfac_loss": 10, "cross": 11, "drift": 12}
EXPORTS = ("kq_workspace_bytes", "kq_hessian_accum", "kq_rotate_in", "kq_hg_sqrt", "kq_rotate_out", "kq_cholinv",
           "kq_quantize_layer", "kq_sensitivity", "kq_unrotate", "kq_layer_loss", "kq_strerror", "kq_last_error",
           "kq_hadamard_order", "kq_version", "kq_allocate_bits", "kq_matvec_quantized",
           "kq_hg_extract", "kq_hg_lowrank", "kq_kfac_loss", "kq_quantize_layer_search",
           "kq_block_order", "kq_permute_blocks", "kq_cross_accum", "kq_drift_target", "kq_matvec_quantized_static")


class KQError(RuntimeError):
    def __init__(self, name: str, status: int, detail: str):
        super().__init__(f"{name} failed: status {status} ({strerror(status)}): {detail}")
        self.status = status


_lib = None
_i64, _vp, _f32, _int, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m post_quantization_03_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "kq_workspace_bytes": (_sz, [_int, _i64, _i64, _i64, _int, _int, _int, _int, _i64]),
        "kq_hessian_accum": (_int, [_vp, _int, _i64, _i64, _i64, ctypes.c_double, ctypes.c_double, _vp, _vp, _sz, _vp]),
        "kq_rotate_in": (_int, [_vp, _int, _i64, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _sz, _vp]),
        "kq_hg_sqrt": (_int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
        "kq_rotate_out": (_int, [_vp, _i64, _i64, _i64, _vp, _int, _i64, _vp, _vp, _sz, _vp]),
        "kq_cholinv": (_int, [_vp, _i64, _i64, ctypes.c_double, _vp, _vp, _vp, _sz, _vp]),
        "kq_quantize_layer": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _int, _int, _int, _vp, _vp, _vp, _vp, _vp, _sz,
                                     _vp]),
        "kq_sensitivity": (_int, [_vp, _i64, _i64, _vp, _int, _i64, _i64, _vp, _vp]),
        "kq_unrotate": (_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _int, _i64, _vp, _i64, _vp, _sz, _vp]),
        "kq_layer_loss": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
        "kq_strerror": (ctypes.c_char_p, [_int]),
        "kq_last_error": (ctypes.c_char_p, []),
        "kq_hadamard_order": (_i64, [_i64, ctypes.POINTER(_i64)]),
        "kq_version": (_int, []),
        "kq_allocate_bits": (_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64), _i64, ctypes.c_double, _int,
                                    _int, ctypes.POINTER(ctypes.c_int32)]),
        "kq_matvec_quantized": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _vp, _vp, _vp, _int, _i64, _vp, _i64, _i64,
                                       _vp, _i64, _vp, _sz, _vp]),
        "kq_matvec_quantized_static": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _vp, _vp, _vp, _int, _i64, _vp,
                                              _i64, _i64, _vp, _i64, _vp]),
        "kq_hg_extract": (_int, [_vp, _i64, _i64, _int, _i64, _vp, _vp]),
        "kq_block_order": (_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
        "kq_cross_accum": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _i64, ctypes.c_double, ctypes.c_double, _vp, _vp,
                                  _sz, _vp]),
        "kq_drift_target": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
        "kq_permute_blocks": (_int, [_vp, _i64, _vp, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp]),
        "kq_quantize_layer_search": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _int, _int, _int, _int, _vp, _vp, _vp,
                                            _vp, _vp, _sz, _vp]),
        "kq_hg_lowrank": (_int, [_vp, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "kq_kfac_loss": (_int, [_vp, _int, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _int, _i64, _vp, _vp, _sz,
                                _vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().kq_strerror(status).decode()


def last_error() -> str:
    return lib().kq_last_error().decode()


def _check(name: str, status: int) -> None:
    if status != 0:
        raise KQError(name, status, last_error())


def _p(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ws(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())


def _xdt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KQ_BF16
    if t.dtype == torch.float32:
        return KQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# ----------------------------------------------------------------------------------- wrappers
def kq_workspace_bytes(op: str, o: int = 0, i: int = 0, n: int = 0, xdt: int = KQ_BF16, bits: int = 0,
                       group: int = 0, form: str = "diag", blk: int = 0) -> int:
    return int(lib().kq_workspace_bytes(OP[op], o, i, n, xdt, bits, group, HG_FORM[form], blk))


def kq_hadamard_order(d: int) -> tuple[int, int]:
    p2 = _i64(0)
    m = lib().kq_hadamard_order(d, ctypes.byref(p2))
    return int(m), int(p2.value)


def kq_hessian_accum(X, H, alpha: float, beta: float, ws=None, stream=None) -> None:
    n, d = X.shape
    w, wb = _ws(ws)
    _check("kq_hessian_accum", lib().kq_hessian_accum(_p(X), _xdt(X), n, d, X.stride(0), alpha, beta, _p(H), w, wb,
                                                      _stream(stream)))


def kq_rotate_in(Win, Wout, HX, sign_in, ws=None, stream=None) -> None:
    o, i = Win.shape
    w, wb = _ws(ws)
    _check("kq_rotate_in", lib().kq_rotate_in(_p(Win), _xdt(Win), Win.stride(0), _p(Wout), Wout.stride(0), o, i,
                                              _p(HX), _p(sign_in), w, wb, _stream(stream)))


def kq_rotate_in_hessian(HX, sign_in, ws=None, stream=None) -> None:
    """kq_rotate_in with no weights: HX <- U^T HX U."""
    i = HX.shape[0]
    w, wb = _ws(ws)
    _check("kq_rotate_in", lib().kq_rotate_in(None, KQ_F32, i, None, i, 0, i, _p(HX), _p(sign_in), w, wb,
                                              _stream(stream)))


def kq_hg_sqrt(HG, form: str, o: int, blk: int, S, Sinv, info, ws=None, stream=None) -> None:
    w, wb = _ws(ws)
    _check("kq_hg_sqrt", lib().kq_hg_sqrt(_p(HG), HG_FORM[form], o, blk, _p(S), _p(Sinv), _p(info), w, wb,
                                          _stream(stream)))


def kq_rotate_out(W, S, form: str, blk: int, sign_out, ws=None, stream=None) -> None:
    o, i = W.shape
    w, wb = _ws(ws)
    _check("kq_rotate_out", lib().kq_rotate_out(_p(W), o, i, W.stride(0), _p(S), HG_FORM[form], blk, _p(sign_out), w,
                                                wb, _stream(stream)))


def kq_cholinv(HX, damp: float, R, info, ws=None, stream=None) -> None:
    i = HX.shape[0]
    w, wb = _ws(ws)
    _check("kq_cholinv", lib().kq_cholinv(_p(HX), i, HX.stride(0), damp, _p(R), _p(info), w, wb, _stream(stream)))


def kq_quantize_layer(W, R, bits: int, group: int, block: int, codes, scale, offset, row_loss=None, ws=None,
                      stream=None) -> None:
    o, i = W.shape
    w, wb = _ws(ws)
    _check("kq_quantize_layer", lib().kq_quantize_layer(_p(W), o, i, W.stride(0), _p(R), R.stride(0), bits, group,
                                                        block, _p(codes), _p(scale), _p(offset), _p(row_loss), w, wb,
                                                        _stream(stream)))


def kq_quantize_layer_search(W, R, bits: int, group: int, block: int, candidates: int, codes, scale, offset,
                             row_loss=None, ws=None, stream=None) -> None:
    o, i = W.shape
    w, wb = _ws(ws)
    _check("kq_quantize_layer_search",
           lib().kq_quantize_layer_search(_p(W), o, i, W.stride(0), _p(R), R.stride(0), bits, group, block, candidates,
                                          _p(codes), _p(scale), _p(offset), _p(row_loss), w, wb, _stream(stream)))


def kq_block_order(H, width: int, order, stream=None) -> None:
    i = H.shape[0]
    _check("kq_block_order", lib().kq_block_order(_p(H), i, H.stride(0), width, _p(order), _stream(stream)))


def kq_permute_blocks(src, dst, width: int, axis: int, perm, stream=None) -> None:
    rows, cols = src.shape
    _check("kq_permute_blocks", lib().kq_permute_blocks(_p(src), src.stride(0), _p(dst), dst.stride(0), rows, cols,
                                                        width, axis, src.element_size(), _p(perm), _stream(stream)))


def kq_cross_accum(A, B, C, alpha: float, beta: float, ws=None, stream=None) -> None:
    n, d = A.shape
    if B.shape != A.shape or B.dtype != A.dtype:
        raise ValueError("kq_cross_accum: A and B must have the same shape and dtype")
    w, wb = _ws(ws)
    _check("kq_cross_accum", lib().kq_cross_accum(_p(A), _p(B), _xdt(A), n, d, A.stride(0), B.stride(0), alpha, beta,
                                                  _p(C), w, wb, _stream(stream)))


def kq_drift_target(W, C, R, Wt, ws=None, stream=None) -> None:
    o, i = W.shape
    w, wb = _ws(ws)
    _check("kq_drift_target", lib().kq_drift_target(_p(W), _xdt(W), W.stride(0), o, i, _p(C), C.stride(0), _p(R),
                                                    R.stride(0), _p(Wt), Wt.stride(0), w, wb, _stream(stream)))


def kq_sensitivity(HX, HG, form: str, o: int, blk: int, score, stream=None) -> None:
    i = HX.shape[0]
    _check("kq_sensitivity", lib().kq_sensitivity(_p(HX), i, HX.stride(0), _p(HG), HG_FORM[form], o, blk, _p(score),
                                                  _stream(stream)))


def kq_unrotate(Q, sign_in, sign_out, Sinv, form: str, blk: int, What, ws=None, stream=None) -> None:
    o, i = Q.shape
    w, wb = _ws(ws)
    _check("kq_unrotate", lib().kq_unrotate(_p(Q), o, i, Q.stride(0), _p(sign_in), _p(sign_out), _p(Sinv),
                                            HG_FORM[form], blk, _p(What), What.stride(0), w, wb, _stream(stream)))


def kq_matvec_quantized(codes, scale, offset, o: int, i: int, bits: int, group: int, sign_in, sign_out, Sinv,
                        form: str, blk: int, X, Y, ws=None, stream=None) -> None:
    """Y (nt x o) = W^ X^T for the tokens in the rows of X (nt x i), from the packed codes."""
    nt = X.shape[0]
    w, wb = _ws(ws)
    _check("kq_matvec_quantized", lib().kq_matvec_quantized(_p(codes), _p(scale), _p(offset), o, i, bits, group,
                                                            _p(sign_in), _p(sign_out), _p(Sinv), HG_FORM[form], blk,
                                                            _p(X), X.stride(0), nt, _p(Y), Y.stride(0), w, wb,
                                                            _stream(stream)))


def kq_matvec_quantized_static(codes, scale, offset, o: int, i: int, bits: int, group: int, sign_in, sign_out, Sinv,
                               form: str, blk: int, X, Y, stream=None) -> None:
    """kq_matvec_quantized on the library's fixed per-device scratch array (no workspace argument)."""
    nt = X.shape[0]
    _check("kq_matvec_quantized_static",
           lib().kq_matvec_quantized_static(_p(codes), _p(scale), _p(offset), o, i, bits, group, _p(sign_in),
                                            _p(sign_out), _p(Sinv), HG_FORM[form], blk, _p(X), X.stride(0), nt, _p(Y),
                                            Y.stride(0), _stream(stream)))


def kq_hg_extract(H, form: str, blk: int, HG, stream=None) -> None:
    o = H.shape[0]
    _check("kq_hg_extract", lib().kq_hg_extract(_p(H), o, H.stride(0), HG_FORM[form], blk, _p(HG), _stream(stream)))


def kq_hg_lowrank(G, k: int, q: int, omega, S, Sinv, HGhat, sigma, info, ws=None, stream=None) -> None:
    n, o = G.shape
    w, wb = _ws(ws)
    _check("kq_hg_lowrank", lib().kq_hg_lowrank(_p(G), n, o, G.stride(0), k, q, _p(omega), _p(S), _p(Sinv),
                                                _p(HGhat), _p(sigma), _p(info), w, wb, _stream(stream)))


def kq_kfac_loss(W, What, HX, HG, form: str, blk: int, loss, ws=None, stream=None) -> None:
    o, i = What.shape
    w, wb = _ws(ws)
    _check("kq_kfac_loss", lib().kq_kfac_loss(_p(W), _xdt(W), W.stride(0), _p(What), What.stride(0), o, i, _p(HX),
                                              HX.stride(0), _p(HG), HG_FORM[form], blk, _p(loss), w, wb,
                                              _stream(stream)))


def kq_layer_loss(W2, Q, HX2, row_loss, loss, ws=None, stream=None) -> None:
    o, i = W2.shape
    w, wb = _ws(ws)
    _check("kq_layer_loss", lib().kq_layer_loss(_p(W2), _p(Q), o, i, W2.stride(0), _p(HX2), HX2.stride(0),
                                                _p(row_loss), _p(loss), w, wb, _stream(stream)))


def kq_allocate_bits(scores, sizes, budget: float = 3.0, bmin: int = 2, bmax: int = 4):
    """Host call: bit-width per sublayer from the sensitivity scores (see include/kq.h)."""
    import numpy as np
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    sz = np.ascontiguousarray(sizes, dtype=np.int64)
    out = np.zeros(len(sc), dtype=np.int32)
    _check("kq_allocate_bits", lib().kq_allocate_bits(sc.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                                      sz.ctypes.data_as(ctypes.POINTER(_i64)), len(sc), budget, bmin,
                                                      bmax, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return out
