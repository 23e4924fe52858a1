"""kq_matvec_quantized_static, the product without a workspace (for callers that cannot allocate), against
kq_matvec_quantized with a workspace: the same kernels, so the outputs must be bit-identical. Two calls in
a row share the library's per-device scratch array, the second with a smaller input; both are also held to
the oracle's bound for the product. Oversized calls are refused before any device work."""
import ctypes

import numpy as np
import pytest

from oracle import kronq as kq
from post_quantization_03_amd import _lib as K
from tests.gpu_util import host, say, to_dev, torch_dev, ws_tensor
from tests.parity import matvec_error_scale


def _static_and_ws(words, sc, mu, o, i, bits, group, s, t, Si, form, blk, X):
    torch, dev = torch_dev()
    nt = X.shape[0]
    args = (torch.from_numpy(words.view(np.int32)).to(dev), to_dev(sc), to_dev(mu), o, i, bits, group,
            to_dev(s, "i8"), to_dev(t, "i8"), to_dev(Si), form, blk)
    Xd = to_dev(X)
    Ys = torch.full((nt, o), float("nan"), dtype=torch.float32, device=dev)
    K.kq_matvec_quantized_static(*args, Xd, Ys)
    ys = host(Ys)
    Yw = torch.full((nt, o), float("nan"), dtype=torch.float32, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("matvec", o, i, nt, form=form, blk=blk))
    ws.fill_(0xFF)  # the workspace variant runs on scratch of other contents than the static array
    K.kq_matvec_quantized(*args, Xd, Yw, ws)
    return ys, host(Yw)


@pytest.mark.gpu
def test_static_matches_workspace_product_twice():
    from tests.test_gpu_ops import matvec_case
    # a large call first (the C2 layer's shape, 8 tokens, full S^-1), then a smaller one (block S^-1,
    # 3 tokens), so the second runs on an array that still holds the first call's contents
    for (form, o, i, bits, group, nt, blk) in (("full", 4096, 4096, 3, 128, 8, 0),
                                               ("block", 256, 1728, 2, 0, 3, 64)):
        say(f"static matvec {form} o={o} i={i} bits={bits} group={group} nt={nt}")
        rng = np.random.default_rng(o + nt)
        words, sc, mu, s, t, Si, X = matvec_case(rng, o, i, bits, group, nt, form, blk)
        ys, yw = _static_and_ws(words, sc, mu, o, i, bits, group, s, t, Si, form, blk, X)
        assert np.all(np.isfinite(ys))
        assert np.array_equal(ys, yw)
        ref = kq.matvec_quantized(words, mu, sc, bits, group, s, t, Si.astype(np.float64), form, X)
        scale = matvec_error_scale(words, mu, sc, bits, group, s, Si, form, X)
        assert np.all(np.linalg.norm(ys - ref, axis=1) <= 1e-5 * scale)


def test_static_refuses_calls_beyond_its_scratch():
    """Host-side: a call needing more than KQ_MATVEC_STATIC_SCRATCH_BYTES returns KQ_EWORKSPACE before
    any device work (stand-in pointers are never dereferenced)."""
    lib = K.lib()
    o, i, nt = 28672, 8192, 64
    need = K.kq_workspace_bytes("matvec", o, i, nt)
    assert need > 32 * 2 ** 20
    p = ctypes.c_void_p(4096)
    st = lib.kq_matvec_quantized_static(p, p, p, o, i, 2, 0, p, p, p, 0, 0, p, i, nt, p, o, None)
    assert st == 6
    assert b"scratch" in lib.kq_last_error()
    assert K.kq_workspace_bytes("matvec", o, i, 16) <= 32 * 2 ** 20
