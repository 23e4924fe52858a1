"""Per-call parity of the HIP library (through the C ABI) against the float64 oracle.

Each call gets the same input bits as the oracle (bf16 / fp32 values widened exactly); inputs that
come from an earlier step are produced by the oracle and rounded to fp32, so a call is checked in
isolation. Sizes span several tiles and a ragged tail.
"""
import numpy as np
import pytest

import synth
from oracle import kronq as kq
from post_quantization_03_amd import _lib as K
from tests.gpu_util import host, say, to_dev, torch_dev, ws_tensor
from tests.parity import TIE, grid_steps, gpu_words_to_codes, hx_tol, matvec_error_scale, rel_fro, replay_compare

pytestmark = pytest.mark.gpu
f32 = np.float32


def spd_f32(rng, d, n=None, spread=1.0):
    n = n or 3 * d
    G = rng.standard_normal((n, d)) * np.exp(spread * rng.standard_normal(d))
    return (G.T @ G / n).astype(f32)


def signs(rng, d):
    return (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)


# ----------------------------------------------------------------------------- H_X
@pytest.mark.parametrize("n,d,dt", [(1000, 200, "bf16"), (4096, 384, "bf16"), (300, 132, "f32"), (64, 8, "bf16"),
                                    (70000, 256, "bf16")])
def test_hessian_accum(n, d, dt):
    torch, dev = torch_dev()
    say(f"hessian n={n} d={d} {dt}")
    sp = synth.scaled(synth.CONFIGS["C2"], n=n, i=d, x_dtype=dt, n_outliers=max(1, d // 100))
    Xs = synth.gen_X(sp)
    ref = kq.hessian(synth.widen(Xs, dt))
    X = to_dev(Xs, dt)
    H = torch.empty((d, d), dtype=torch.float64, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("hessian", 0, d, n, K.KQ_BF16 if dt == "bf16" else K.KQ_F32))
    K.kq_hessian_accum(X, H, 1.0 / n, 0.0, ws)
    Hg = host(H)
    err = rel_fro(Hg, ref)
    say(f"  H_X rel err {err:.2e}")
    assert np.array_equal(Hg, Hg.T)
    tol = hx_tol(n) if dt == "bf16" else 1e-12
    assert err <= tol
    assert np.abs(Hg - ref).max() <= tol * np.diag(ref).max()


def test_hessian_accumulates_batches():
    torch, dev = torch_dev()
    sp = synth.scaled(synth.CONFIGS["C2"], n=3000, i=256)
    Xs = synth.gen_X(sp)
    ref = kq.hessian(synth.widen(Xs, "bf16"))
    X = to_dev(Xs, "bf16")
    H = torch.empty((256, 256), dtype=torch.float64, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("hessian", 0, 256, 3000))
    for k0, beta in ((0, 0.0), (1000, 1.0), (2000, 1.0)):
        K.kq_hessian_accum(X[k0:k0 + 1000], H, 1.0 / 3000, beta, ws)
    assert rel_fro(host(H), ref) <= hx_tol(1000)


# ----------------------------------------------------------------------------- input rotation
@pytest.mark.parametrize("o,i,wdt,with_h", [(40, 256, "f32", True), (33, 320, "bf16", True), (16, 224, "f32", True),
                                            (8, 384, "bf16", True), (24, 1728, "bf16", True), (5, 11008, "bf16", False),
                                            (3, 5120, "f32", True)])
def test_rotate_in(o, i, wdt, with_h):
    torch, dev = torch_dev()
    say(f"rotate_in o={o} i={i} {wdt} H={with_h}")
    rng = np.random.default_rng(o * 7 + i)
    W64 = rng.standard_normal((o, i)) * 0.02
    Ws = synth.f32_to_bf16_bits(W64.astype(f32)) if wdt == "bf16" else W64.astype(f32)
    s = signs(rng, i)
    H64 = spd_f32(rng, i, n=i + 16).astype(np.float64) if with_h else None
    W1_ref = kq.rotate_in_weights(synth.widen(Ws, wdt), s)
    Win = to_dev(Ws, wdt)
    Wout = torch.empty((o, i), dtype=torch.float32, device=dev)
    Hd = to_dev(H64, "f64") if with_h else None
    ws = ws_tensor(K.kq_workspace_bytes("rotate_in", o, i))
    K.kq_rotate_in(Win, Wout, Hd, to_dev(s, "i8"), ws)
    assert rel_fro(host(Wout), W1_ref) <= 2e-6
    if with_h:
        H2_ref = kq.rotate_in_hessian(H64, s)
        assert rel_fro(host(Hd), H2_ref) <= 1e-13


# ----------------------------------------------------------------------------- H_G square root
@pytest.mark.parametrize("form,o,blk", [("diag", 1000, 0), ("block", 384, 128), ("full", 256, 0), ("full", 200, 0),
                                        ("block", 256, 64), ("full", 1024, 0), ("full", 1000, 0), ("full", 2048, 0)])
def test_hg_sqrt(form, o, blk):
    """Full form: 256, 1024 and 2048 (whole 128-wide blocks) run the sweep with pivots launched ahead
    that wait on the device; 200 and 1000 (a ragged last block) run the queue-wait pipeline."""
    torch, dev = torch_dev()
    say(f"hg_sqrt {form} o={o} blk={blk}")
    if form == "diag":
        hg = synth.gen_HG(synth.scaled(synth.CONFIGS["C3"], o=o))
    elif form == "block":
        hg = synth.gen_HG(synth.scaled(synth.CONFIGS["C4"], o=o, hg_blk=blk))
    else:
        hg = synth.gen_HG(synth.scaled(synth.CONFIGS["C2"], o=o, hg_ng=2 * o))
    S_ref, Si_ref = kq.hg_sqrt(hg.astype(np.float64), form)
    S = torch.empty(hg.shape, dtype=torch.float32, device=dev)
    Si = torch.empty_like(S)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("hg_sqrt", o, 0, 0, form=form, blk=blk))
    K.kq_hg_sqrt(to_dev(hg), form, o, blk, S, Si, info, ws)
    assert int(host(info)[0]) == 0
    assert rel_fro(host(S), S_ref) <= 1e-6
    assert rel_fro(host(Si), Si_ref) <= 1e-6


@pytest.mark.parametrize("cond,dense", [(1e2, True), (1e6, True), (1e12, False)])
def test_hg_sqrt_step_counts(cond, dense):
    """Full-form H_G whose spectral bounds need 5, 6 and 7 Denman-Beavers steps (the last, a diagonal
    matrix with cond 1e12, is exactly positive definite in fp32): the call reads the first step's
    bounds back and launches the remaining steps itself, so each must come out converged."""
    torch, dev = torch_dev()
    o = 256
    rng = np.random.default_rng(11)
    lam = np.logspace(0.0, -np.log10(cond), o)
    if dense:
        Q, _ = np.linalg.qr(rng.standard_normal((o, o)))
        hg = ((Q * lam) @ Q.T).astype(f32)
        hg = 0.5 * (hg + hg.T)
    else:
        hg = np.diag(lam).astype(f32)
    say(f"hg_sqrt cond={cond:.0e} dense={dense}")
    S_ref, Si_ref = kq.hg_sqrt(hg.astype(np.float64), "full")
    S = torch.empty(hg.shape, dtype=torch.float32, device=dev)
    Si = torch.empty_like(S)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("hg_sqrt", o, 0, 0, form="full"))
    K.kq_hg_sqrt(to_dev(hg), "full", o, 0, S, Si, info, ws)
    assert int(host(info)[0]) == 0
    assert rel_fro(host(S), S_ref) <= 1e-6
    assert rel_fro(host(Si), Si_ref) <= 1e-6


def test_hg_sqrt_repeated_calls_identical():
    """Repeated calls on one workspace (with eager work and host synchronisations between them) and a
    call on a second workspace give bit-identical roots, equal to the oracle's: the result depends
    on no state left by an earlier call (sweep queues, events, scratch)."""
    torch, dev = torch_dev()
    o = 384
    hg = synth.gen_HG(synth.scaled(synth.CONFIGS["C2"], o=o, hg_ng=2 * o))
    S_ref, _ = kq.hg_sqrt(hg.astype(np.float64), "full")
    HG = to_dev(hg)
    nb = K.kq_workspace_bytes("hg_sqrt", o, 0, 0, form="full")
    ws1, ws2 = ws_tensor(nb), ws_tensor(nb)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    outs = []
    for ws in (ws1, ws1, ws2, ws1):
        S = torch.empty((o, o), dtype=torch.float32, device=dev)
        K.kq_hg_sqrt(HG, "full", o, 0, S, None, info, ws)
        junk = torch.randn((o, o), device=dev) @ torch.randn((o, o), device=dev)  # eager work in between
        torch.cuda.synchronize()
        assert int(host(info)[0]) == 0
        outs.append(host(S).copy())
        del junk
    for S in outs[1:]:
        assert np.array_equal(S, outs[0])
    assert rel_fro(outs[0], S_ref) <= 1e-6


_FALLBACK_SCRIPT = r"""
import os
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import synth
from oracle import kronq as kq
from post_quantization_03_amd import _lib as K
dev = torch.device("cuda:0")
o = 512
hg = synth.gen_HG(synth.scaled(synth.CONFIGS["C2"], o=o, hg_ng=2 * o))
S_ref, _ = kq.hg_sqrt(hg.astype(np.float64), "full")
HG = torch.from_numpy(hg).to(dev)
ws = torch.empty(K.kq_workspace_bytes("hg_sqrt", o, 0, 0, form="full"), dtype=torch.uint8, device=dev)


def call(tag):
    S = torch.empty((o, o), dtype=torch.float32, device=dev)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    K.kq_hg_sqrt(HG, "full", o, 0, S, None, info, ws)
    note = K.last_error()
    torch.cuda.synchronize()
    err = np.linalg.norm(S.cpu().numpy().astype(np.float64) - S_ref) / np.linalg.norm(S_ref)
    inf = int(info.cpu()[0])
    print(f"{tag}: info {inf} rel err {err:.3e} notice {note!r}", flush=True)
    return inf, err, note


# every wait cut to one poll: each call notices after its first step and redoes itself with queue
# waits (nothing is kept between calls, so the second call does the same)
os.environ["KQ_SWEEP_WAIT_POLLS"] = "1"
for c in range(2):
    inf, err, note = call(f"cut from step 0, call {c}")
    assert inf == 0 and err <= 1e-6 and "ran out" in note
# cut only from the second step on: the first step's read-back sees no run-out, a later wait runs out,
# and the call reports info = -1 (S invalid; the caller re-issues the call)
os.environ["KQ_SWEEP_WAIT_FROM_STEP"] = "1"
inf, err, note = call("cut from step 1")
assert inf == -1 and "ran out" not in note
# limits restored: the re-issued call matches, with no notice
del os.environ["KQ_SWEEP_WAIT_POLLS"], os.environ["KQ_SWEEP_WAIT_FROM_STEP"]
inf, err, note = call("re-issued")
assert inf == 0 and err <= 1e-6 and note == ""
print("OK", flush=True)
"""


def test_hg_sqrt_falls_back_when_device_wait_runs_out():
    """The sweep's pivot kernels are launched ahead and wait on the device, in a bounded loop, for the
    other queue's gather. With that bound cut to one poll (KQ_SWEEP_WAIT_POLLS, in a child process) the
    first waits run out: the square root notices at its read-back after the first step, redoes the call
    with queue waits, leaves a notice in kq_last_error and still matches the oracle with info 0; a
    second call does the same (no state is kept between calls). Cut only from the second step on
    (KQ_SWEEP_WAIT_FROM_STEP), a later wait runs out and the call reports info = -1; re-issued with the
    limits restored it matches, with no notice."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = {k: v for k, v in os.environ.items() if not k.startswith("KQ_SWEEP_WAIT")}
    r = subprocess.run([sys.executable, "-c", _FALLBACK_SCRIPT, root], env=env, capture_output=True, text=True,
                       timeout=180)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
    assert "OK" in r.stdout


def test_hg_sqrt_reports_not_positive_definite():
    torch, dev = torch_dev()
    for form, hg in (("full", -np.eye(128, dtype=f32)), ("diag", -np.ones(64, f32))):
        o = hg.shape[0]
        S = torch.empty(hg.shape, dtype=torch.float32, device=dev)
        info = torch.zeros(1, dtype=torch.int32, device=dev)
        ws = ws_tensor(K.kq_workspace_bytes("hg_sqrt", o, 0, 0, form=form))
        K.kq_hg_sqrt(to_dev(hg), form, o, 0, S, None, info, ws)
        assert int(host(info)[0]) > 0


# ----------------------------------------------------------------------------- output transform
@pytest.mark.parametrize("form,o,i,blk", [("diag", 256, 128, 0), ("diag", 320, 64, 0), ("full", 256, 192, 0),
                                          ("block", 384, 128, 128), ("full", 224, 64, 0), ("block", 5120, 16, 128)])
def test_rotate_out(form, o, i, blk):
    torch, dev = torch_dev()
    say(f"rotate_out {form} o={o} i={i}")
    rng = np.random.default_rng(o + i)
    W = (rng.standard_normal((o, i)) * 0.02).astype(f32)
    t = signs(rng, o)
    if form == "diag":
        S = np.exp(rng.standard_normal(o)).astype(f32)
    elif form == "block":
        S = np.stack([spd_f32(rng, blk) for _ in range(o // blk)])
    else:
        S = spd_f32(rng, o)
    ref = kq.rotate_out(W.astype(np.float64), S.astype(np.float64), form, t)
    Wd = to_dev(W)
    ws = ws_tensor(K.kq_workspace_bytes("rotate_out", o, i, form=form, blk=blk))
    K.kq_rotate_out(Wd, to_dev(S), form, blk, to_dev(t, "i8"), ws)
    assert rel_fro(host(Wd), ref) <= 2e-6


# ----------------------------------------------------------------------------- damped factor
@pytest.mark.parametrize("i", [200, 384, 1000, 128, 6200, 333, 6147])
def test_cholinv(i):
    """Widths of 6144 and more take the two-level panel factorisation (6200: a ragged last panel and
    diagonal block). Even widths run each step's update and the next diagonal sweep in one launch
    (200, 1000, 6200: ragged last tiles); odd widths (333, 6147) keep separate launches."""
    torch, dev = torch_dev()
    say(f"cholinv i={i}")
    sp = synth.scaled(synth.CONFIGS["C2"], n=(4 if i < 4096 else 2) * i, i=i, n_outliers=max(1, i // 100))
    H64 = kq.hessian(synth.widen(synth.gen_X(sp), "bf16"))
    H, _ = kq.damped(H64, 0.01)
    R_ref = kq.inverse_upper_factor(H)
    R = torch.empty((i, i), dtype=torch.float32, device=dev)
    info = torch.full((1,), 7, dtype=torch.int32, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("cholinv", 0, i))
    K.kq_cholinv(to_dev(H64, "f64"), 0.01, R, info, ws)
    Rg = host(R).astype(np.float64)
    assert int(host(info)[0]) == 0
    assert np.all(np.tril(Rg, -1) == 0)
    err = rel_fro(Rg, R_ref)
    say(f"  R rel err {err:.3e} cond {np.linalg.cond(H):.3e}")
    assert err <= 1e-6


def test_cholinv_concurrent_with_hg_sqrt():
    """The damped factor computed while the H_G square root runs on another stream equals the serial
    result bit for bit (every work-group of the in-place panel product owns whole rows: with two
    column tiles per row block, a late tile read what its neighbour had already overwritten)."""
    torch, dev = torch_dev()
    i, o = 2048, 2048
    say(f"cholinv i={i} concurrent with hg_sqrt o={o}")
    sp = synth.scaled(synth.CONFIGS["C2"], n=2 * i, i=i, o=o, hg_ng=2 * o, n_outliers=4)
    Hd = to_dev(kq.hessian(synth.widen(synth.gen_X(sp), "bf16")), "f64")
    HG = to_dev(synth.gen_HG(sp))
    ws = ws_tensor(K.kq_workspace_bytes("cholinv", 0, i))
    ws_s = ws_tensor(K.kq_workspace_bytes("hg_sqrt", o, 0, 0, form="full"))
    S = torch.empty((o, o), dtype=torch.float32, device=dev)
    R0 = torch.empty((i, i), dtype=torch.float32, device=dev)
    info = torch.zeros(4, dtype=torch.int32, device=dev)
    K.kq_cholinv(Hd, 0.01, R0, info[0:1], ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    for rep in range(3):
        R = torch.empty_like(R0)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            K.kq_hg_sqrt(HG, "full", o, 0, S, None, info[1:2], ws_s)
        K.kq_cholinv(Hd, 0.01, R, info[2:3], ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert host(info).tolist()[:3] == [0, 0, 0]
        assert torch.equal(R, R0), f"repeat {rep}"


def test_cholinv_panel_calls_side_by_side():
    """Two panel factorisations enqueued on two streams at once equal the same calls made one after the
    other, bit for bit."""
    torch, dev = torch_dev()
    i = 6400
    say(f"cholinv i={i} twice, side by side")
    Hs, Rs, R0s = [], [], []
    for k in range(2):
        sp = synth.scaled(synth.CONFIGS["C2"], n=2 * i, i=i, n_outliers=8, layer=k)
        Hs.append(to_dev(kq.hessian(synth.widen(synth.gen_X(sp), "bf16")), "f64"))
    ws = [ws_tensor(K.kq_workspace_bytes("cholinv", 0, i)) for _ in range(2)]
    info = torch.zeros(4, dtype=torch.int32, device=dev)
    for k in range(2):
        R0s.append(torch.empty((i, i), dtype=torch.float32, device=dev))
        K.kq_cholinv(Hs[k], 0.01, R0s[k], info[k:k + 1], ws[k])
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    for k in range(2):
        Rs.append(torch.empty_like(R0s[k]))
        streams[k].wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(streams[k]):
            K.kq_cholinv(Hs[k], 0.01, Rs[k], info[2 + k:3 + k], ws[k])
    for st in streams:
        torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    assert host(info).tolist() == [0, 0, 0, 0]
    for k in range(2):
        assert torch.equal(Rs[k], R0s[k])


def test_cholinv_reports_not_positive_definite():
    torch, dev = torch_dev()
    i = 256
    H = -np.eye(i)
    R = torch.empty((i, i), dtype=torch.float32, device=dev)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    K.kq_cholinv(to_dev(H, "f64"), 0.0, R, info, ws_tensor(K.kq_workspace_bytes("cholinv", 0, i)))
    assert int(host(info)[0]) > 0


# ----------------------------------------------------------------------------- sweep
@pytest.mark.parametrize("o,i,bits,group", [(37, 384, 3, 128), (37, 384, 4, 0), (64, 256, 2, 128), (20, 512, 2, 0),
                                            (16, 256, 3, 64), (9, 256, 8, 32), (130, 1024, 3, 128),
                                            (130, 2048, 3, 128), (48, 2560, 2, 0),
                                            (16400, 256, 2, 0), (16400, 128, 3, 128)])
def test_quantize_layer(o, i, bits, group):
    """From 16384 rows the sweep runs on row panels side by side (16400: four panels, the last one
    shorter and not a multiple of the 16-row work-group). 2048 and 2560 columns take two and three
    1024-column super-blocks, each followed by its deep (K = 1024) trailing update."""
    torch, dev = torch_dev()
    say(f"quantize o={o} i={i} b={bits} g={group}")
    tall = o > 4096
    sp = synth.scaled(synth.CONFIGS["C2"], o=o, i=i, n=4 * i, hg_ng=2 * o if 64 <= o <= 4096 else 256, n_outliers=2,
                      hg_form="diag" if tall else "full")
    d = synth.layer_inputs(sp)
    hg = d["HG"] if 64 <= o <= 4096 else np.ones(o, f32)
    form = "full" if 64 <= o <= 4096 else "diag"
    r = kq.quantize_layer(synth.widen(d["X"], "bf16"), synth.widen(d["W"], "bf16"), hg.astype(np.float64), form,
                          d["s"], d["t"], bits, group, verify=False, rotate_out_on=False)
    W2 = r["W2"].astype(f32)
    R = r["R"].astype(f32)
    Wd = to_dev(W2)
    codes = torch.empty((o, i * bits // 32), dtype=torch.int32, device=dev)
    ng = i // group if group else 1
    scale = torch.empty((o, ng), dtype=torch.float32, device=dev)
    offset = torch.empty((o, ng), dtype=torch.float32, device=dev)
    rl = torch.empty((o,), dtype=torch.float32, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("quantize", o, i))
    K.kq_quantize_layer(Wd, to_dev(R), bits, group, 128, codes, scale, offset, rl, ws)
    words = host(codes)
    gc = gpu_words_to_codes(words, bits, i)
    cmp = replay_compare(gc, W2.astype(np.float64), R.astype(np.float64), bits, group, 128)
    say(f"  replays={cmp['replays']} fail={cmp['fail'][:3]}")
    assert not cmp["fail"]
    oc = np.stack([cmp["codes"][k] for k in range(o)])
    assert np.array_equal(kq.pack(oc, bits), words.view(np.uint32))
    Q = np.stack([cmp["Q"][k] for k in range(o)])
    assert rel_fro(host(Wd), Q) <= 1e-5
    loss = np.array([cmp["row_loss"][k] for k in range(o)])
    assert np.allclose(host(rl), loss, rtol=1e-3, atol=1e-12)
    mu = np.stack([cmp["mu"][k] for k in range(o)])
    sc = np.stack([cmp["scale"][k] for k in range(o)])
    assert rel_fro(host(offset), mu) <= 1e-4 and rel_fro(host(scale), sc) <= 1e-4
    dmu, ds = grid_steps(host(offset), host(scale), mu, sc, bits)
    say(f"  grid parameters: |d mu|/s {dmu:.2e}, L |d s|/s {ds:.2e} grid steps")
    assert dmu <= TIE and ds <= 2 * TIE


@pytest.mark.parametrize("o,i,bits,group,cands", [(37, 384, 3, 128, 500), (20, 512, 2, 0, 500), (16, 256, 4, 32, 64),
                                                  (64, 256, 2, 64, 500)])
def test_quantize_layer_search(o, i, bits, group, cands):
    """Hessian-aware grids: the GPU's candidate at every grid is replayed in the oracle, must be the
    oracle's minimum up to 1e-4 relative (the objective is summed in fp32 on the GPU) and never worse
    than min-max; then codes, words, w^, row loss and grid parameters as for the min-max sweep."""
    torch, dev = torch_dev()
    say(f"quantize search o={o} i={i} b={bits} g={group} candidates={cands}")
    tall = o > 4096
    sp = synth.scaled(synth.CONFIGS["C2"], o=o, i=i, n=4 * i, hg_ng=2 * o if 64 <= o <= 4096 else 256, n_outliers=2,
                      hg_form="diag" if tall else "full")
    d = synth.layer_inputs(sp)
    hg = d["HG"] if 64 <= o <= 4096 else np.ones(o, f32)
    form = "full" if 64 <= o <= 4096 else "diag"
    r = kq.quantize_layer(synth.widen(d["X"], "bf16"), synth.widen(d["W"], "bf16"), hg.astype(np.float64), form,
                          d["s"], d["t"], bits, group, verify=False, rotate_out_on=False)
    W2 = r["W2"].astype(f32)
    R = r["R"].astype(f32)
    Wd = to_dev(W2)
    codes = torch.empty((o, i * bits // 32), dtype=torch.int32, device=dev)
    ng = i // group if group else 1
    scale = torch.empty((o, ng), dtype=torch.float32, device=dev)
    offset = torch.empty((o, ng), dtype=torch.float32, device=dev)
    rl = torch.empty((o,), dtype=torch.float32, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("quantize", o, i))
    K.kq_quantize_layer_search(Wd, to_dev(R), bits, group, 128, cands, codes, scale, offset, rl, ws)
    words = host(codes)
    gc = gpu_words_to_codes(words, bits, i)
    sc_gpu = host(scale)
    cmp = replay_compare(gc, W2.astype(np.float64), R.astype(np.float64), bits, group, 128, search=cands,
                         gpu_scale=sc_gpu)
    say(f"  replays={cmp['replays']} fail={cmp['fail'][:3]}")
    assert not cmp["fail"]
    shrunk = 0
    for k in range(o):
        obj, ch = cmp["objectives"][k], cmp["chosen"][k]
        for g in range(ng):
            best = obj[g].min()
            assert obj[g, ch[g]] <= best * (1 + 1e-4) + 1e-30, (k, g, ch[g], obj[g].argmin())
            assert obj[g, ch[g]] <= obj[g, -1] * (1 + 1e-6) + 1e-30
            shrunk += int(ch[g] < cands - 1)
    say(f"  grids narrower than min-max: {shrunk} of {o * ng}")
    oc = np.stack([cmp["codes"][k] for k in range(o)])
    assert np.array_equal(kq.pack(oc, bits), words.view(np.uint32))
    Q = np.stack([cmp["Q"][k] for k in range(o)])
    assert rel_fro(host(Wd), Q) <= 1e-5
    loss = np.array([cmp["row_loss"][k] for k in range(o)])
    assert np.allclose(host(rl), loss, rtol=1e-3, atol=1e-12)
    mu = np.stack([cmp["mu"][k] for k in range(o)])
    sc = np.stack([cmp["scale"][k] for k in range(o)])
    assert rel_fro(host(offset), mu) <= 1e-4 and rel_fro(sc_gpu, sc) <= 1e-4


# ----------------------------------------------------------------------------- sensitivity, unrotate, loss
@pytest.mark.parametrize("form", ["diag", "block", "full"])
def test_sensitivity(form):
    torch, dev = torch_dev()
    rng = np.random.default_rng(3)
    i, o = 300, 256
    H = spd_f32(rng, i)
    hg = {"diag": np.exp(rng.standard_normal(o)).astype(f32),
          "block": np.stack([spd_f32(rng, 64) for _ in range(4)]),
          "full": spd_f32(rng, o)}[form]
    score = torch.empty(1, dtype=torch.float64, device=dev)
    K.kq_sensitivity(to_dev(H, "f64"), to_dev(hg), form, o, 64, score)
    ref = kq.sensitivity(H.astype(np.float64), hg.astype(np.float64), form)
    assert abs(host(score)[0] / ref - 1) <= 1e-12


@pytest.mark.parametrize("form,o,i,blk", [("full", 256, 320, 0), ("diag", 320, 256, 0), ("block", 256, 1728, 128)])
def test_unrotate_and_loss(form, o, i, blk):
    torch, dev = torch_dev()
    say(f"unrotate {form} o={o} i={i}")
    rng = np.random.default_rng(o * i)
    Q = (rng.standard_normal((o, i)) * 0.02).astype(f32)
    W2 = (Q + rng.standard_normal((o, i)) * 0.002).astype(f32)
    s, t = signs(rng, i), signs(rng, o)
    if form == "diag":
        Si = np.exp(rng.standard_normal(o)).astype(f32)
    elif form == "block":
        Si = np.stack([spd_f32(rng, blk) for _ in range(o // blk)])
    else:
        Si = spd_f32(rng, o)
    ref = kq.unrotate(Q.astype(np.float64), s, t, Si.astype(np.float64), form)
    What = torch.empty((o, i), dtype=torch.float32, device=dev)
    ws = ws_tensor(max(K.kq_workspace_bytes("unrotate", o, i, form=form, blk=blk), K.kq_workspace_bytes("loss", o, i)))
    K.kq_unrotate(to_dev(Q), to_dev(s, "i8"), to_dev(t, "i8"), to_dev(Si), form, blk, What, ws)
    assert rel_fro(host(What), ref) <= 2e-6
    H = spd_f32(rng, i)
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    rl = torch.empty(o, dtype=torch.float64, device=dev)
    K.kq_layer_loss(to_dev(W2), to_dev(Q), to_dev(H, "f64"), rl, loss, ws)
    lref = kq.rotated_loss(W2.astype(np.float64), Q.astype(np.float64), H.astype(np.float64))
    assert abs(host(loss)[0] / lref.sum() - 1) <= 1e-5
    assert np.allclose(host(rl), lref, rtol=1e-4)


# ----------------------------------------------------------------------------- inference-side product
MATVEC_TOL = 1e-5


def matvec_case(rng, o, i, bits, group, nt, form, blk):
    """Random packed codes (any word is a valid stream), group scales s > 0 and offsets about
    -s 2^(b-1) as a min-max grid would give, tokens with log-normal channel scales."""
    g = group if group else i
    words = rng.integers(0, 2 ** 32, size=(o, i * bits // 32), dtype=np.uint64).astype(np.uint32)
    sc = (0.002 * np.exp(0.5 * rng.standard_normal((o, i // g)))).astype(f32)
    mu = (-sc * (2 ** (bits - 1)) * (1 + 0.1 * rng.standard_normal((o, i // g)))).astype(f32)
    s, t = signs(rng, i), signs(rng, o)
    if form == "diag":
        Si = np.exp(rng.standard_normal(o)).astype(f32)
    elif form == "block":
        Si = np.stack([spd_f32(rng, blk) for _ in range(o // blk)])
    else:
        Si = spd_f32(rng, o)
    X = (rng.standard_normal((nt, i)) * np.exp(rng.standard_normal(i))).astype(f32)
    return words, sc, mu, s, t, Si, X


def run_matvec(words, sc, mu, o, i, bits, group, s, t, Si, form, blk, X):
    torch, dev = torch_dev()
    nt = X.shape[0]
    Y = torch.full((nt, o), float("nan"), dtype=torch.float32, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("matvec", o, i, nt, form=form, blk=blk))
    K.kq_matvec_quantized(torch.from_numpy(words.view(np.int32)).to(dev), to_dev(sc), to_dev(mu), o, i, bits, group,
                          to_dev(s, "i8"), to_dev(t, "i8"), to_dev(Si), form, blk, to_dev(X), Y, ws)
    return host(Y)


@pytest.mark.parametrize("form,o,i,bits,group,nt,blk", [
    ("diag", 256, 256, 4, 128, 1, 0),
    ("full", 320, 512, 3, 128, 3, 0),
    ("block", 256, 1728, 2, 0, 5, 64),
    ("diag", 40, 5120, 5, 64, 8, 0),       # ragged rows, ragged last column slice
    ("diag", 96, 4096, 6, 32, 11, 0),      # two token passes (8 + 3), column slices
    ("full", 64, 13824, 7, 128, 2, 0),     # Paley input order, six slices
    ("block", 128, 2048, 8, 256, 4, 128),
    ("full", 128, 256, 4, 32, 9, 0),       # more than 8 tokens: S^{-1} through the general GEMM
    ("block", 96, 256, 3, 128, 2, 6),      # block size not a multiple of 4: general GEMM
    ("diag", 96, 1024, 5, 128, 16, 0),     # matrix-core product: 16 tokens, generic unpacking
    ("full", 128, 768, 6, 0, 17, 0),       # matrix-core product: two token passes, per-row grids
    ("diag", 200, 2560, 2, 128, 6, 0),     # matrix-core product: ragged row blocks, 5 slices
    ("diag", 64, 1024, 8, 128, 8, 0),      # matrix-core product: 8-bit codes (signed shift)
    ("full", 64, 512, 4, 0, 12, 0),        # matrix-core product: 4-bit codes, per-row grids
    ("diag", 48, 1536, 3, 256, 5, 0),      # matrix-core product: 3-bit codes, groups over two windows
    ("diag", 200, 2560, 2, 128, 3, 0),     # same shape at 3 tokens: the VALU product
])
def test_matvec_quantized(form, o, i, bits, group, nt, blk):
    say(f"matvec {form} o={o} i={i} bits={bits} group={group} nt={nt}")
    rng = np.random.default_rng(o * 31 + i + bits)
    words, sc, mu, s, t, Si, X = matvec_case(rng, o, i, bits, group, nt, form, blk)
    Y = run_matvec(words, sc, mu, o, i, bits, group, s, t, Si, form, blk, X)
    ref = kq.matvec_quantized(words, mu, sc, bits, group, s, t, Si.astype(np.float64), form, X)
    scale = matvec_error_scale(words, mu, sc, bits, group, s, Si, form, X)
    err = np.linalg.norm(Y - ref, axis=1)
    assert np.all(np.isfinite(Y))
    assert np.all(err <= MATVEC_TOL * scale), (err / scale).max()


def test_argument_errors_are_reported():
    torch, dev = torch_dev()
    W = torch.zeros((8, 100), dtype=torch.float32, device=dev)
    R = torch.zeros((100, 100), dtype=torch.float32, device=dev)
    with pytest.raises(K.KQError) as e:
        K.kq_quantize_layer(W, R, 3, 128, 128, W, W, W, None, ws_tensor(1 << 20))
    assert e.value.status == 2   # i not a multiple of 128
    with pytest.raises(K.KQError) as e:
        K.kq_rotate_in(W, W, None, torch.ones(100, dtype=torch.int8, device=dev), ws_tensor(1 << 20))
    assert e.value.status == 4   # 100 = 25 * 4: no Hadamard order


def test_matvec_quantized_graph_replays():
    """The product captured in a HIP graph (as a decode loop would replay it): every replay, with
    eager work and synchronisations between replays, equals the eager call."""
    torch, dev = torch_dev()
    o, i, bits, group, nt, form, blk = 256, 4096, 3, 128, 2, "full", 0
    rng = np.random.default_rng(77)
    words, sc, mu, s, t, Si, X = matvec_case(rng, o, i, bits, group, nt, form, blk)
    args = [torch.from_numpy(words.view(np.int32)).to(dev), to_dev(sc), to_dev(mu), o, i, bits, group,
            to_dev(s, "i8"), to_dev(t, "i8"), to_dev(Si), form, blk]
    x = to_dev(X)
    ws = ws_tensor(K.kq_workspace_bytes("matvec", o, i, nt, form=form, blk=blk))
    y_eager = torch.empty((nt, o), dtype=torch.float32, device=dev)
    K.kq_matvec_quantized(*args, x, y_eager, ws)
    ref = host(y_eager).copy()
    y = torch.full((nt, o), float("nan"), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            K.kq_matvec_quantized(*args, x, y, ws)
    torch.cuda.current_stream().wait_stream(side)
    for k in range(3):
        y.fill_(float("nan"))
        K.kq_matvec_quantized(*args, x, y_eager, ws)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), ref), k


# ----------------------------------------------------------------------------- H_G preparation, K-FAC loss
@pytest.mark.parametrize("form,blk", [("full", 0), ("block", 64), ("diag", 0)])
def test_hg_extract(form, blk):
    torch, dev = torch_dev()
    rng = np.random.default_rng(4)
    o = 320
    H = spd_f32(rng, o).astype(np.float64) * (1 + 1e-9 * rng.standard_normal((o, o)))
    H = (H + H.T) / 2
    want = kq.hg_forms(H, form, blk).astype(np.float32)
    out = torch.empty(want.shape, dtype=torch.float32, device=dev)
    K.kq_hg_extract(to_dev(H, "f64"), form, blk, out)
    assert np.array_equal(host(out), want)


@pytest.mark.parametrize("o,n,k,q", [(512, 2048, 64, 2), (384, 1000, 200, 0), (256, 300, 128, 4)])
def test_hg_lowrank(o, n, k, q):
    torch, dev = torch_dev()
    say(f"hg_lowrank o={o} n={n} k={k} q={q}")
    rng = np.random.default_rng(o + k)
    scales = np.abs(rng.standard_t(3, size=o)) + 0.05
    G = (rng.standard_normal((n, o)) * scales).astype(f32)
    omega = rng.standard_normal((o, k)).astype(f32)
    ref = kq.hg_lowrank(G.astype(np.float64), k, q, omega.astype(np.float64))
    S, Si, Hh = (torch.empty((o, o), dtype=torch.float32, device=dev) for _ in range(3))
    sig = torch.empty(2, dtype=torch.float64, device=dev)
    info = torch.full((1,), -1, dtype=torch.int32, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("hg_lowrank", o, k, n))
    K.kq_hg_lowrank(to_dev(G), k, q, to_dev(omega), S, Si, Hh, sig, info, ws)
    assert int(host(info)[0]) == 0
    s_gpu = host(sig)
    assert abs(s_gpu[0] / ref["sigma"] - 1) <= 1e-9 and abs(s_gpu[1] / ref["trH"] - 1) <= 1e-12
    assert rel_fro(host(Hh), ref["Hhat"]) <= 1e-6
    assert rel_fro(host(S), ref["S"]) <= 1e-6
    assert rel_fro(host(Si), ref["Sinv"]) <= 1e-6


def test_hg_lowrank_reports_rank_loss():
    """G of rank k/2 < k: the range basis of H Omega cannot have rank k (info = 1)."""
    torch, dev = torch_dev()
    rng = np.random.default_rng(8)
    o, n, k = 256, 512, 64
    G = (rng.standard_normal((n, k // 2)) @ rng.standard_normal((k // 2, o))).astype(f32)
    S = torch.empty((o, o), dtype=torch.float32, device=dev)
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("hg_lowrank", o, k, n))
    K.kq_hg_lowrank(to_dev(G), k, 1, to_dev(rng.standard_normal((o, k)).astype(f32)), S, None, None, None, info, ws)
    assert int(host(info)[0]) == 1


@pytest.mark.parametrize("form,o,i,blk,wdt", [("full", 256, 320, 0, "f32"), ("block", 256, 384, 64, "bf16"),
                                              ("diag", 200, 256, 0, "f32")])
def test_kfac_loss(form, o, i, blk, wdt):
    torch, dev = torch_dev()
    rng = np.random.default_rng(o * i)
    W = (rng.standard_normal((o, i)) * 0.02).astype(f32)
    if wdt == "bf16":
        W = synth.bf16_round(W)
    What = (W + rng.standard_normal((o, i)) * 0.003).astype(f32)
    HX = spd_f32(rng, i).astype(np.float64)
    if form == "diag":
        HG = np.exp(rng.standard_normal(o)).astype(f32)
    elif form == "block":
        HG = np.stack([spd_f32(rng, blk) for _ in range(o // blk)])
    else:
        HG = spd_f32(rng, o)
    ref = kq.kfac_loss(W.astype(np.float64), What.astype(np.float64), HX, HG.astype(np.float64), form)
    Wd = to_dev(synth.f32_to_bf16_bits(W), "bf16") if wdt == "bf16" else to_dev(W)
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    ws = ws_tensor(K.kq_workspace_bytes("kfac_loss", o, i, form=form, blk=blk))
    K.kq_kfac_loss(Wd, to_dev(What), to_dev(HX, "f64"), to_dev(HG), form, blk, loss, ws)
    assert abs(host(loss)[0] / ref - 1) <= 1e-10


# ----------------------------------------------------------------------------- trace-ordered blocks
def test_block_order_and_permute():
    torch, dev = torch_dev()
    rng = np.random.default_rng(31)
    i, o, nb = 1024, 40, 8
    A = rng.standard_normal((3 * i, i)) * np.exp(rng.standard_normal(i))
    H = A.T @ A / (3 * i)
    order = torch.empty(2 * nb, dtype=torch.int32, device=dev)
    Hd = to_dev(H, "f64")
    K.kq_block_order(Hd, 128, order)
    want = kq.block_trace_order(H, 128)
    got = host(order)
    assert list(got[:nb]) == list(want) and list(got[nb:]) == list(np.argsort(want))
    p = kq.block_perm_index(want, 128)
    Ht, Hp = torch.empty_like(Hd), torch.empty_like(Hd)
    K.kq_permute_blocks(Hd, Ht, 128, 0, order[:nb])
    K.kq_permute_blocks(Ht, Hp, 128, 1, order[:nb])
    assert np.array_equal(host(Hp), H[np.ix_(p, p)])
    W = rng.standard_normal((o, i)).astype(f32)
    Wd, Wp, Wb = to_dev(W), torch.empty((o, i), dtype=torch.float32, device=dev), torch.empty((o, i), dtype=torch.float32, device=dev)
    K.kq_permute_blocks(Wd, Wp, 128, 0, order[:nb])
    assert np.array_equal(host(Wp), W[:, p])
    K.kq_permute_blocks(Wp, Wb, 128, 0, order[nb:])
    assert np.array_equal(host(Wb), W)


@pytest.mark.parametrize("bits,group,search", [(3, 128, 500), (2, 0, 0), (4, 32, 64)])
def test_layer_trace_order(bits, group, search):
    """The layer with blocks in trace order (and the grid search): GPU block order equal to the
    oracle's; codes and packed words compared on the permuted problem (near-tie and candidate
    replays as for the plain sweep); w^ and the grids back in natural order."""
    from post_quantization_03_amd.layer import LayerCfg, quantize_layer
    torch, dev = torch_dev()
    o, i = 48, 640
    say(f"trace order o={o} i={i} b={bits} g={group} search={search}")
    sp = synth.scaled(synth.CONFIGS["C3"], o=o, i=i, n=4 * i, n_outliers=2)
    d = synth.layer_inputs(sp)
    X, W = to_dev(d["X"], "bf16"), to_dev(d["W"], "bf16")
    cfg = LayerCfg(bits=bits, group=group, form="diag", search=search, order="trace")
    out = quantize_layer(X, W, to_dev(d["HG"]), to_dev(d["s"], "i8"), to_dev(d["t"], "i8"), cfg)
    assert host(out["info"]).tolist() == [0, 0]
    ref = kq.quantize_layer(synth.widen(d["X"], "bf16"), synth.widen(d["W"], "bf16"), d["HG"].astype(np.float64),
                            "diag", d["s"], d["t"], bits, group, verify=False, search=search, order="trace")
    nb = i // 128
    order = host(out["order"])[:nb]
    assert list(order) == list(ref["order"])
    p = kq.block_perm_index(order, 128)
    words = host(out["codes"])
    gc = gpu_words_to_codes(words, bits, i)
    sc = host(out["scale"])
    gsc = sc[:, kq.block_perm_index(order, 128 // group)] if group else sc
    # the permuted problem with the GPU's fp32 factor
    W2p = ref["W2"][:, p]
    Rg = host(out["R"]).astype(np.float64)
    cmp = replay_compare(gc[:, p], W2p, Rg, bits, group, 128, search=search, gpu_scale=gsc if search else None)
    say(f"  replays={cmp['replays']} fail={cmp['fail'][:3]}")
    assert not cmp["fail"]
    oc = np.stack([cmp["codes"][k] for k in range(o)])
    inv = np.argsort(p)
    assert np.array_equal(kq.pack(oc[:, inv], bits), words.view(np.uint32))
    Q = np.stack([cmp["Q"][k] for k in range(o)])[:, inv]
    assert rel_fro(host(out["Q"]), Q) <= 1e-5
    assert rel_fro(Rg, ref["R_perm"]) <= 1e-5


# ----------------------------------------------------------------------------- input drift
@pytest.mark.parametrize("n,d,dt", [(10000, 256, "bf16"), (3000, 320, "f32")])
def test_cross_accum(n, d, dt):
    torch, dev = torch_dev()
    rng = np.random.default_rng(n + d)
    A = (rng.standard_normal((n, d)) * np.exp(rng.standard_normal(d))).astype(f32)
    B = (A + 0.1 * rng.standard_normal((n, d))).astype(f32)
    if dt == "bf16":
        A, B = synth.bf16_round(A), synth.bf16_round(B)
        Ad, Bd = to_dev(synth.f32_to_bf16_bits(A), "bf16"), to_dev(synth.f32_to_bf16_bits(B), "bf16")
    else:
        Ad, Bd = to_dev(A), to_dev(B)
    C = to_dev(np.eye(d), "f64")
    K.kq_cross_accum(Ad, Bd, C, 1.0 / n, 0.5, ws_tensor(K.kq_workspace_bytes("cross", 0, d, n)))
    ref = A.astype(np.float64).T @ B.astype(np.float64) / n + 0.5 * np.eye(d)
    assert rel_fro(host(C), ref) <= 1e-12


def test_drift_target():
    torch, dev = torch_dev()
    rng = np.random.default_rng(5)
    o, i, n = 96, 384, 2000
    X = rng.standard_normal((n, i)) * np.exp(rng.standard_normal(i))
    Xt = X + 0.05 * rng.standard_normal((n, i))
    W = (rng.standard_normal((o, i)) * 0.02).astype(f32)
    dr = kq.drift_target(W, X, Xt)
    H, lam = kq.damped(dr["H"])
    R = kq.inverse_upper_factor(H).astype(f32)
    ref = W.astype(np.float64) @ dr["C"] @ (R.astype(np.float64).T @ R.astype(np.float64))
    Wt = torch.empty((o, i), dtype=torch.float32, device=dev)
    K.kq_drift_target(to_dev(W), to_dev(dr["C"], "f64"), to_dev(R), Wt, ws_tensor(K.kq_workspace_bytes("drift", o, i)))
    assert rel_fro(host(Wt), ref) <= 1e-7
    assert rel_fro(host(Wt), dr["W"]) <= 1e-4     # R rounded to fp32 on both sides of the first check


@pytest.mark.parametrize("bits,group", [(3, 128), (2, 0)])
def test_layer_drift(bits, group):
    """The layer with drifted inputs: target W* and H~ from the GPU against the oracle, codes on the
    sweep's input with near-tie replays, w^ in rotated coordinates."""
    from post_quantization_03_amd.layer import LayerCfg, quantize_layer
    torch, dev = torch_dev()
    o, i = 64, 512
    say(f"drift o={o} i={i} b={bits} g={group}")
    sp = synth.scaled(synth.CONFIGS["C2"], o=o, i=i, n=4 * i, hg_ng=2 * o, n_outliers=2)
    d = synth.layer_inputs(sp)
    Xt = synth.gen_X_drift(sp)
    cfg = LayerCfg(bits=bits, group=group, form="full")
    out = quantize_layer(to_dev(d["X"], "bf16"), to_dev(d["W"], "bf16"), to_dev(d["HG"]), to_dev(d["s"], "i8"),
                         to_dev(d["t"], "i8"), cfg, X_drift=to_dev(Xt, "bf16"))
    assert host(out["info"]).tolist() == [0, 0]
    ref = kq.quantize_layer(synth.widen(d["X"], "bf16"), synth.widen(d["W"], "bf16"), d["HG"].astype(np.float64),
                            "full", d["s"], d["t"], bits, group, verify=False, Xt=synth.widen(Xt, "bf16"))
    assert rel_fro(host(out["H"]), ref["HX2"]) <= hx_tol(sp.n)
    words = host(out["codes"])
    gc = gpu_words_to_codes(words, bits, i)
    Rg = host(out["R"]).astype(np.float64)
    cmp = replay_compare(gc, ref["W2"], Rg, bits, group, 128)
    say(f"  replays={cmp['replays']} fail={cmp['fail'][:3]}")
    assert not cmp["fail"]
    Q = np.stack([cmp["Q"][k] for k in range(o)])
    assert rel_fro(host(out["Q"]), Q) <= 1e-4
