"""Host-side checks of the C-ABI library: it loads, exports every symbol the header declares, and its
host logic (workspace sizing, Hadamard orders, argument validation before any device work) behaves.
No GPU needed: nothing here launches a kernel."""
import os
import re

import numpy as np
import pytest

from oracle import hadamard as hd
from post_quantization_03_amd import _lib as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "kq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = K.lib()
    names = header_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(K.EXPORTS)
    assert lib.kq_version() >= 1


def test_hadamard_orders_agree_with_oracle():
    for d in [1, 4, 8, 12, 20, 28, 108, 256, 344, 4096, 5120, 8192, 11008, 13824, 28672, 1728, 224, 320, 1376]:
        assert K.kq_hadamard_order(d) == hd.decompose(d), d
    for d in [100, 3 * 5 * 17, 6]:
        assert K.kq_hadamard_order(d)[0] == 0


def test_workspace_sizes():
    # C2 shapes: hessian split partials, hg_sqrt fp64 Denman-Beavers buffers, full S apply buffer
    assert K.kq_workspace_bytes("hessian", 4096, 4096, 65536, K.KQ_BF16) > 0
    assert K.kq_workspace_bytes("hessian", 256, 256, 2048, K.KQ_F32) >= 2048 * 256 * 8   # fp64 copy of fp32 X
    hg = K.kq_workspace_bytes("hg_sqrt", 4096, 0, 0, form="full")
    assert hg >= 2 * 2 * 4096 * 4096 * 8      # Y, Z and their sweep buffers in fp64
    assert K.kq_workspace_bytes("hg_sqrt", 4096, 0, 0, form="diag") == 0
    assert K.kq_workspace_bytes("rotate_out", 4096, 4096, form="full") >= 4096 * 4096 * 4
    assert K.kq_workspace_bytes("rotate_in", 4096, 4096) < 4096       # power of two: only the empty P slot
    assert K.kq_workspace_bytes("rotate_in", 5120, 13824) >= 13824 * 13824 * 4
    assert K.kq_workspace_bytes("cholinv", 0, 4096) >= 2 * 4096 * 4096 * 4
    assert K.kq_workspace_bytes("quantize", 28672, 8192) >= 28672 * 512 * 4


def test_host_validation_without_device_work():
    lib = K.lib()
    # null pointers and bad sizes are rejected before anything is enqueued
    assert lib.kq_cholinv(None, 16, 16, 0.01, None, None, None, 0, None) == 1
    assert lib.kq_quantize_layer(None, 4, 128, 128, None, 128, 3, 128, 128, None, None, None, None, None, 0, None) == 1
    assert lib.kq_hessian_accum(None, 1, 4, 8, 8, 1.0, 0.0, None, None, 0, None) == 1
    assert lib.kq_sensitivity(None, 8, 8, None, 0, 8, 0, None, None) == 1
    assert lib.kq_strerror(6) == b"workspace too small"
    assert b"null" in lib.kq_last_error()


def test_product_path_has_no_fallback():
    """The binding loads only the in-tree HIP library and never imports the oracle."""
    src = open(os.path.join(ROOT, "post_quantization_03_amd", "_lib.py")).read()
    src += open(os.path.join(ROOT, "post_quantization_03_amd", "layer.py")).read()
    assert "from oracle" not in src and "import oracle" not in src


def test_allocation_matches_oracle():
    """The library's host allocator against the oracle's (independent implementations of one reading)."""
    import numpy as np
    from oracle import alloc
    import synth
    rng = np.random.default_rng(5)
    sizes = np.array([o * i for (_, o, i, _) in synth.C5_SUBLAYERS] * 32, dtype=np.int64)
    for trial in range(5):
        scores = np.exp(4 * rng.standard_normal(len(sizes)))
        got = K.kq_allocate_bits(scores, sizes, 3.0, 2, 4)
        want = alloc.allocate(scores, sizes, 3.0, 2, 4)
        assert np.array_equal(got, want)
        assert np.dot(got, sizes) <= 3.0 * sizes.sum()
    assert np.array_equal(K.kq_allocate_bits(np.ones(7), np.full(7, 100)), np.full(7, 3))


def test_gradient_rows_match_the_full_hg_draws():
    """gen_G draws the same gradient rows that gen_HG accumulates (full form)."""
    import synth
    sp = synth.scaled(synth.CONFIGS["C2"], o=96, hg_ng=5000)
    G = synth.gen_G(sp).astype(np.float64)
    H = synth.gen_HG(sp).astype(np.float64)
    assert np.abs(G.T @ G / sp.hg_ng - H).max() <= 1e-6 * np.abs(H).max()
    assert synth.gen_omega(sp, 8).shape == (96, 8)


HELPERS = {"kq_workspace_bytes", "kq_strerror", "kq_last_error", "kq_version"}
SECTIONS = ("Background", "Method", "Key idea", "Prior limitations", "Limitations", "Where this paper sits",
            "Goal", "Sparks", "Weight scales and rounding", "abstract", "Comparison")


def header_comments():
    """{function name: the comment right before its declaration} for every call in include/kq.h."""
    txt = open(os.path.join(ROOT, "include", "kq.h")).read()
    out = {}
    for m in re.finditer(r"/\*(.*?)\*/\s*(?:kq_status|const char\*|int64_t|int|size_t)\s+(kq_[a-z_0-9]+)\s*\(",
                         txt, flags=re.S):
        out[m.group(2)] = " ".join(re.sub(r"\n\s*\*", " ", m.group(1)).split())
    return out


def test_every_method_call_cites_a_page_section():
    """Each call of the method (every declaration but the helpers) names the page section that
    defines its operation in the comment above it."""
    comments = header_comments()
    calls = [n for n in header_functions() if n not in HELPERS and n not in ("kq_strerror", "kq_last_error")]
    missing = [n for n in calls if n not in comments]
    assert not missing, f"declarations without a comment: {missing}"
    # the entry point without a workspace names the callers it is for instead of a passage
    no_alloc = [n for n in calls if "callers that cannot allocate" in comments[n]]
    assert no_alloc == ["kq_matvec_quantized_static"]
    uncited = [n for n in calls if n not in no_alloc and
               ("page" not in comments[n] or not any(sec in comments[n] for sec in SECTIONS))]
    assert not uncited, f"calls whose comment names no page section: {uncited}"


def test_header_states_the_library_owned_resources():
    """The conventions block says what the library keeps per device and which calls read back."""
    txt = open(os.path.join(ROOT, "include", "kq.h")).read()
    conv = txt[txt.index("Conventions shared by every call"):txt.index("#ifndef KQ_H")]
    assert "never allocates device memory" in conv
    assert "two queues" in conv and "kq_hg_sqrt" in conv and "capturing" in conv
    src = "".join(open(os.path.join(ROOT, "post_quantization_03_amd", "csrc", f)).read()
                  for f in os.listdir(os.path.join(ROOT, "post_quantization_03_amd", "csrc")))
    src = re.sub(r"//[^\n]*", "", src)
    assert "hipMalloc" not in src and "hipFree" not in src
