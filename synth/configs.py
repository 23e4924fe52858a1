"""Registry of the five synthetic workloads and their seeded generators.

Every array is drawn in float64 from ``numpy.random.Generator(PCG64(SeedSequence(
[cfg, layer, sub, tag])))``, rounded to fp32 (round-to-nearest-even), and, where
the workload stores bf16, rounded again to bf16 (round-to-nearest-even on the
fp32 bit pattern). bf16 arrays are returned as their raw ``uint16`` bit patterns
so that every consumer widens exactly the same bits.

Shapes and value distributions stand in for the LLaMA layers and calibration
statistics that the KronQ pages evaluate on (LLaMA-2-7B q_proj, LLaMA-2-13B
down_proj, LLaMA-3-70B up_proj, a 32-layer LLaMA-2-7B stack); no model weights or
text data are used.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Iterator

import numpy as np

TAG_W, TAG_X, TAG_G, TAG_S, TAG_T, TAG_OUT, TAG_OMEGA, TAG_DRIFT = 0, 1, 2, 3, 4, 5, 6, 7


def rng(cfg: int, layer: int, sub: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, layer, sub, tag])))


# ----------------------------------------------------------------------------- storage rounding
def f32_to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round-to-nearest-even. Inputs must be finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit pattern (uint16) -> fp32, exact."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a) -> np.ndarray:
    """Round to bf16 and widen back to fp32 (exact widening)."""
    return bf16_to_f32(f32_to_bf16_bits(a))


# ----------------------------------------------------------------------------- workload spec
@dataclass(frozen=True)
class LayerSpec:
    name: str
    cfg: int            # 1..5
    layer: int
    sub: int            # sublayer index (seed for W and H_G)
    o: int              # output channels (rows of W)
    i: int              # input channels (columns of W)
    n: int              # calibration tokens
    x_dtype: str        # "f32" | "bf16"
    w_dtype: str        # "f32" | "bf16"
    w_std: float
    x_recipe: str       # "lognormal" | "relu"
    x_sigma: float      # log-normal sigma of the per-channel scales
    n_outliers: int     # channels multiplied by 20
    x_sub: int          # seed index of the activation (several sublayers may share one input)
    hg_form: str        # "diag" | "block" | "full"
    hg_lo: float = -1.5     # diag: log10 of the smallest entry
    hg_span: float = 3.0    # diag: decades spanned
    hg_mag: bool = False    # diag: multiply by a per-sublayer magnitude exp(N(0,1))
    hg_blk: int = 128       # block: block size
    hg_ng: int = 0          # block/full: gradient samples
    bits: int = 4
    group: int = 0          # 0 = one grid per output row, else group size along the input axis
    block: int = 128        # column block of the solver
    damp: float = 0.01

    @property
    def weights(self) -> int:
        return self.o * self.i


CONFIGS = {
    "C1": LayerSpec("C1 256x256 W4 per-row", 1, 0, 0, 256, 256, 2048, "f32", "f32", 0.02,
                    "lognormal", 1.0, 4, 0, "diag", -1.5, 3.0, bits=4, group=0),
    "C2": LayerSpec("C2 4096x4096 W3 g128 (q_proj)", 2, 0, 0, 4096, 4096, 65536, "bf16", "bf16", 0.02,
                    "lognormal", 1.5, 41, 0, "full", hg_ng=16384, bits=3, group=128),
    "C3": LayerSpec("C3 5120x13824 W2 g128 (down_proj)", 3, 0, 0, 5120, 13824, 32768, "bf16", "bf16", 0.015,
                    "relu", 0.0, 0, 0, "diag", -2.0, 4.0, bits=2, group=128),
    "C4": LayerSpec("C4 28672x8192 W2 per-row (up_proj)", 4, 0, 0, 28672, 8192, 16384, "bf16", "bf16", 0.01,
                    "lognormal", 2.0, 0, 0, "block", hg_blk=128, hg_ng=512, bits=2, group=0),
}

# 32-layer stack: (name, o, i, input index)
C5_SUBLAYERS = (("q", 4096, 4096, 0), ("k", 4096, 4096, 0), ("v", 4096, 4096, 0), ("o", 4096, 4096, 1),
                ("gate", 11008, 4096, 2), ("up", 11008, 4096, 2), ("down", 4096, 11008, 3))
# input index -> (name, width, recipe)
C5_INPUTS = ((("attn_in", 4096, "lognormal")), (("o_in", 4096, "lognormal")),
             (("mlp_in", 4096, "lognormal")), (("down_in", 11008, "relu")))
C5_LAYERS = 32
C5_TOKENS = 8192


def c5_specs(layer: int, bits=None) -> list[LayerSpec]:
    """The 7 sublayers of one layer of the 32-layer stack. ``bits`` maps sublayer -> bit-width."""
    out = []
    for sub, (nm, o, i, xin) in enumerate(C5_SUBLAYERS):
        recipe = C5_INPUTS[xin][2]
        out.append(LayerSpec(f"C5 L{layer}.{nm} {o}x{i}", 5, layer, sub, o, i, C5_TOKENS, "bf16", "bf16", 0.02,
                             recipe, 1.5 if recipe == "lognormal" else 0.0,
                             round(0.01 * i) if recipe == "lognormal" else 0, xin, "diag", -1.5, 3.0, hg_mag=True,
                             bits=3 if bits is None else int(bits[sub]), group=128))
    return out


def scaled(spec: LayerSpec, **kw) -> LayerSpec:
    """Same recipe at another size (used for small parity cases)."""
    return replace(spec, **kw)


# ----------------------------------------------------------------------------- generators
def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    return f32_to_bf16_bits(a32) if dtype == "bf16" else a32


def gen_W(spec: LayerSpec) -> np.ndarray:
    """Weights o x i, row-major. fp32 array, or uint16 bf16 bits."""
    g = rng(spec.cfg, spec.layer, spec.sub, TAG_W)
    return _store(g.standard_normal((spec.o, spec.i)) * spec.w_std, spec.w_dtype)


def _x_channel_scales(spec: LayerSpec, g: np.random.Generator) -> np.ndarray | None:
    if spec.x_recipe == "relu":
        return None
    sc = np.exp(spec.x_sigma * g.standard_normal(spec.i))
    if spec.n_outliers:
        go = rng(spec.cfg, spec.layer, spec.x_sub, TAG_OUT)
        idx = go.choice(spec.i, size=spec.n_outliers, replace=False)
        sc[idx] *= 20.0
    return sc


def gen_X_chunks(spec: LayerSpec, rows: int | None = None, chunk: int = 4096) -> Iterator[np.ndarray]:
    """Calibration activations n x i in row chunks (the first ``rows`` tokens if given).

    The draws are sequential, so any prefix of the token axis is the same whatever
    ``rows`` or ``chunk`` is.
    """
    n = spec.n if rows is None else min(rows, spec.n)
    g = rng(spec.cfg, spec.layer, spec.x_sub, TAG_X)
    sc = _x_channel_scales(spec, g)
    done = 0
    while done < n:
        m = min(chunk, n - done)
        z = g.standard_normal((m, spec.i))
        if spec.x_recipe == "relu":
            x = np.maximum(z + 0.2533, 0.0)
        else:
            x = z * sc[None, :]
        yield _store(x, spec.x_dtype)
        done += m


def gen_X_drift(spec: LayerSpec, rows: int | None = None, rel: float = 0.05) -> np.ndarray:
    """Drifted calibration inputs X~ (what the layer sees once earlier layers are quantized), n x i in
    the storage type: the same draws as gen_X plus independent noise of `rel` times each channel's
    scale (1 for the ReLU recipe), added before the storage rounding."""
    n = spec.n if rows is None else min(rows, spec.n)
    g = rng(spec.cfg, spec.layer, spec.x_sub, TAG_X)
    gd = rng(spec.cfg, spec.layer, spec.x_sub, TAG_DRIFT)
    sc = _x_channel_scales(spec, g)
    dt = np.uint16 if spec.x_dtype == "bf16" else np.float32
    out = np.empty((n, spec.i), dtype=dt)
    done = 0
    while done < n:
        m = min(4096, n - done)
        z = g.standard_normal((m, spec.i))
        x = np.maximum(z + 0.2533, 0.0) if spec.x_recipe == "relu" else z * sc[None, :]
        noise = gd.standard_normal((m, spec.i)) * (1.0 if sc is None else sc[None, :])
        out[done:done + m] = _store(x + rel * noise, spec.x_dtype)
        done += m
    return out


def gen_X(spec: LayerSpec, rows: int | None = None) -> np.ndarray:
    n = spec.n if rows is None else min(rows, spec.n)
    dt = np.uint16 if spec.x_dtype == "bf16" else np.float32
    out = np.empty((n, spec.i), dtype=dt)
    r = 0
    for c in gen_X_chunks(spec, rows):
        out[r:r + c.shape[0]] = c
        r += c.shape[0]
    return out


def gen_HG(spec: LayerSpec) -> np.ndarray:
    """Output-gradient covariance in its storage form, fp32.

    diag:  o entries, log-normal profile spanning ``hg_span`` decades.
    block: (o/blk, blk, blk) dense SPD blocks G_b^T G_b / n_g.
    full:  o x o dense SPD G^T G / n_g with Student-t(3) channel scales.
    """
    g = rng(spec.cfg, spec.layer, spec.sub, TAG_G)
    if spec.hg_form == "diag":
        z = g.standard_normal(spec.o)
        r = (z - z.min()) / (z.max() - z.min())
        h = 10.0 ** (spec.hg_lo + spec.hg_span * r)
        if spec.hg_mag:
            h = h * np.exp(g.standard_normal())
        return h.astype(np.float32)
    if spec.hg_form == "block":
        b = spec.hg_blk
        nb = spec.o // b
        out = np.empty((nb, b, b), dtype=np.float32)
        for k in range(nb):
            sc = np.exp(g.standard_normal(b))
            G = g.standard_normal((spec.hg_ng, b)) * sc[None, :]
            H = G.T @ G / spec.hg_ng
            out[k] = (0.5 * (H + H.T)).astype(np.float32)
        return out
    if spec.hg_form == "full":
        o = spec.o
        sc = np.abs(g.standard_t(3, size=o))
        H = np.zeros((o, o))
        left = spec.hg_ng
        while left > 0:
            m = min(4096, left)
            G = g.standard_normal((m, o)) * sc[None, :]
            H += G.T @ G
            left -= m
        H /= spec.hg_ng
        return (0.5 * (H + H.T)).astype(np.float32)
    raise ValueError(spec.hg_form)


def gen_G(spec: LayerSpec) -> np.ndarray:
    """The gradient rows behind a full-form H_G (hg_ng x o, fp32): the same draws as gen_HG, so
    G^T G / hg_ng is gen_HG's matrix up to the fp32 rounding of G."""
    if spec.hg_form != "full":
        raise ValueError("gradient rows are generated for the full form only")
    g = rng(spec.cfg, spec.layer, spec.sub, TAG_G)
    o = spec.o
    sc = np.abs(g.standard_t(3, size=o))
    out = np.empty((spec.hg_ng, o), dtype=np.float32)
    r0 = 0
    while r0 < spec.hg_ng:
        m = min(4096, spec.hg_ng - r0)
        out[r0:r0 + m] = (g.standard_normal((m, o)) * sc[None, :]).astype(np.float32)
        r0 += m
    return out


def gen_omega(spec: LayerSpec, k: int) -> np.ndarray:
    """Gaussian test matrix (o x k, fp32) for the randomised range finder of a low-rank H_G."""
    return rng(spec.cfg, spec.layer, spec.sub, TAG_OMEGA).standard_normal((spec.o, k)).astype(np.float32)


def gen_signs(spec: LayerSpec) -> tuple[np.ndarray, np.ndarray]:
    """Random +-1 sign vectors (s for the input side, t for the output side), int8."""
    s = (rng(spec.cfg, spec.layer, spec.x_sub, TAG_S).integers(0, 2, size=spec.i) * 2 - 1).astype(np.int8)
    t = (rng(spec.cfg, spec.layer, spec.sub, TAG_T).integers(0, 2, size=spec.o) * 2 - 1).astype(np.int8)
    return s, t


def layer_inputs(spec: LayerSpec, x_rows: int | None = None) -> dict:
    """All inputs of one layer: X, W, H_G, signs (storage types)."""
    s, t = gen_signs(spec)
    return {"X": gen_X(spec, x_rows), "W": gen_W(spec), "HG": gen_HG(spec), "s": s, "t": t}


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64, exact."""
    return (bf16_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)).astype(np.float64)
