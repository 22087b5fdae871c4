"""CPU tests of the C-ABI library's host side (no GPU work is enqueued).

* the library loads and exports every function include/forge.h declares;
* per-step scalars, composed into each optimizer's per-element update the way
  the kernels apply them, reproduce the oracle's update (float32 scalars: 1e-6);
* the host build of the counter-hash RNG and stochastic rounding agree with the
  oracle's independent implementation bit for bit;
* argument validation returns the documented status before any launch.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from oracle import optim, rounding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def f():
    import optimizer_gemm_amd as forge
    return forge


def _declared():
    text = open(os.path.join(ROOT, "include", "forge.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(forge_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(f):
    names = _declared()
    assert "forge_linear_wgrad_step" in names and "forge_linear_dgrad" in names
    lib = f.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in forge.h but not exported"
    out = os.popen(f"nm -D --defined-only {f.forge.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_status_strings(f):
    for code in range(0, -10, -1):
        assert f.status_str(code) not in ("", "unknown status")
    assert f.status_str(42) == "unknown status"
    assert f.version() >= 100


def test_default_hyper_matches_sweep_defaults(f):
    for opt in optim.OPTIMIZERS:
        d = f.default_hyper(opt)
        o = optim.hyper(opt)
        for k in ("lr", "beta1", "beta2", "eps", "weight_decay", "momentum", "dampening", "alpha", "lr_decay",
                  "momentum_decay"):
            assert d[k] == o[k], (opt, k)


def _kernel_update(opt, s, g, w, m, v):
    """The kernels' per-element arithmetic, restated in float64 from the library's scalars."""
    if opt == "adamw":
        w = w * s["decay"]
        m = s["b1"] * m + s["omb1"] * g
        v = s["b2"] * v + s["omb2"] * g * g
        w = w - s["step_size"] * m / (np.sqrt(v) * s["inv_sqrt_bc2"] + s["eps"])
    elif opt == "sgd":
        w = w - s["lr"] * (g + s["wd"] * w)
    elif opt == "sgd_momentum":
        d = g + s["wd"] * w
        m = s["b1"] * m + s["omb1"] * d
        w = w - s["lr"] * ((d + s["c_m"] * m) if s["flag"] else m)
    elif opt == "lion":
        c = s["b1"] * m + s["omb1"] * g
        w = w * s["decay"] - s["lr"] * np.sign(c)
        m = s["b2"] * m + s["omb2"] * g
    elif opt == "rmsprop":
        d = g + s["wd"] * w
        v = s["b2"] * v + s["omb2"] * d * d
        w = w - s["lr"] * d / (np.sqrt(v) + s["eps"])
    elif opt == "adagrad":
        d = g + s["wd"] * w
        v = v + d * d
        w = w - s["lr"] * d / (np.sqrt(v) + s["eps"])
    elif opt == "nadam":
        d = g + s["wd"] * w
        m = s["b1"] * m + s["omb1"] * d
        v = s["b2"] * v + s["omb2"] * d * d
        w = w - (s["c_g"] * d + s["c_m"] * m) / (np.sqrt(v) * s["inv_sqrt_bc2"] + s["eps"])
    elif opt == "radam":
        d = g + s["wd"] * w
        m = s["b1"] * m + s["omb1"] * d
        v = s["b2"] * v + s["omb2"] * d * d
        w = w - (s["step_size"] * m / (np.sqrt(v) + s["eps"]) if s["flag"] else s["step_size"] * m)
    return w, m, v


@pytest.mark.parametrize("opt", optim.OPTIMIZERS)
@pytest.mark.parametrize("over", [{}, {"weight_decay": 0.02}, {"nesterov": True, "dampening": 0.1},
                                  {"lr_decay": 0.1}])
def test_step_scalars_reproduce_oracle_update(f, opt, over):
    over = {k: v for k, v in over.items() if not (opt != "sgd_momentum" and k in ("nesterov", "dampening"))
            and not (opt != "adagrad" and k == "lr_decay")}
    hp = optim.hyper(opt, **over)
    gh = dict(hp, nesterov=int(hp["nesterov"]), stochastic_round=1)
    rng = np.random.default_rng(0)
    w = rng.standard_normal(500) * 0.02
    m = np.zeros(500)
    v = np.zeros(500)
    wr, mr, vr = w.copy(), m.copy(), v.copy()
    slots = optim.SLOTS[opt]
    for t in range(1, 13):
        g = rng.standard_normal(500) * 1e-2
        s = f.step_scalars(opt, gh, t)
        w, m, v = _kernel_update(opt, s, g, w, m, v)
        wr, mr_, vr_ = optim.update(opt, wr, g, mr if "m" in slots else None, vr if "v" in slots else None, hp, t)
        mr = mr_ if mr_ is not None else mr
        vr = vr_ if vr_ is not None else vr
        # float32 scalars: update error ~1e-6 of an lr-sized step, decay factor error ~1e-7 of |w|
        assert np.all(np.abs(w - wr) <= 1e-5 * hp["lr"] + 2e-7 * np.abs(wr)), (opt, t)
        wr = w.copy()  # teacher-force: next step starts from the same state
        # float32 scalars: relative 1e-6 with a floor at 0.1 rms (cancellation in beta*m + (1-beta)*g)
        if "m" in slots:
            np.testing.assert_allclose(m, mr, rtol=1e-6, atol=1e-6 * 0.1 * np.sqrt(np.mean(mr * mr)))
            mr = m.copy()
        if "v" in slots:
            np.testing.assert_allclose(v, vr, rtol=1e-6, atol=1e-6 * 0.1 * np.sqrt(np.mean(vr * vr)))
            vr = v.copy()


def test_radam_branch_flag(f):
    flags = [f.step_scalars("radam", None, t)["flag"] for t in range(1, 9)]
    assert flags == [0, 0, 0, 0, 0, 1, 1, 1]


def test_host_rng_matches_oracle(f):
    rng = np.random.default_rng(1)
    for _ in range(300):
        seed = int(rng.integers(0, 2 ** 63)) * 2 + int(rng.integers(0, 2))
        step = int(rng.integers(1, 1 << 20))
        idx = int(rng.integers(0, 2 ** 32))
        assert f.rand16(seed, step, idx) == int(rounding.rand16(seed, step, np.array([idx], dtype=np.uint64))[0])


def test_host_sr_matches_oracle(f):
    rng = np.random.default_rng(2)
    xs = np.concatenate([(rng.standard_normal(2000) * 10.0 ** rng.integers(-38, 38, 2000)).astype(np.float32),
                         np.array([np.inf, -np.inf, np.nan, -0.0, 0.0, np.finfo(np.float32).max], np.float32)])
    rs = rng.integers(0, 65536, size=xs.size)
    ref = rounding.sr_bf16(xs, rs)
    got = np.array([f.sr_bf16(float(x), int(r)) for x, r in zip(xs, rs)], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


# --------------------------------------------------------------------------- validation
# Fake, never-dereferenced addresses: every call below must fail validation before a launch.
# They are not run where a GPU is visible, so a validation bug can never launch on them.
def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


cpu_only = pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation tests run only without a GPU")


def _t(f, ptr, dt, rows, cols, ld=None, scale=None):
    return f.forge.ForgeTensor(ptr, dt, 0, rows, cols, cols if ld is None else ld, scale)


def _call_step(f, X, dY, W, m, v, opt="adamw", step=1, hyper=None):
    h = f.make_hyper(opt if isinstance(opt, str) else "adamw", **(hyper or {}))
    r = lambda x: ctypes.byref(x) if x is not None else None  # noqa: E731
    return f.lib().forge_linear_wgrad_step(r(X), r(dY), r(W), r(m), r(v), f.forge.OPT_ID[opt] if isinstance(opt, str)
                                          else opt, ctypes.byref(h), step, 0, None)


@cpu_only
def test_validation_errors(f):
    F32, BF16, I8, U8 = 0, 1, 2, 3
    A = 0x10000000
    B = 0x20000000
    C = 0x30000000
    Mp = 0x40000000
    Vp = 0x50000000
    S1, S2 = 0x60000000, 0x70000000
    X = _t(f, A, BF16, 64, 256)
    dY = _t(f, B, BF16, 64, 128)
    W = _t(f, C, BF16, 128, 256)
    m = _t(f, Mp, F32, 128, 256)
    v = _t(f, Vp, F32, 128, 256)
    E = f.forge
    assert _call_step(f, None, dY, W, m, v) == -1
    assert _call_step(f, X, dY, W, None, v) == -1                       # AdamW needs m
    assert _call_step(f, X, _t(f, B, BF16, 63, 128), W, m, v) == -2      # T mismatch
    assert _call_step(f, X, dY, _t(f, C, BF16, 128, 248), m, v) == -2     # in mismatch
    assert _call_step(f, X, dY, W, _t(f, Mp, F32, 127, 256), v) == -2     # state shape
    assert _call_step(f, _t(f, A, F32, 64, 256), dY, W, m, v) == -3      # mixed io dtypes
    assert _call_step(f, X, dY, W, _t(f, Mp, BF16, 128, 256), v) == -3    # mixed bf16 / f32 moments
    mb, vb = _t(f, Mp, BF16, 128, 256), _t(f, Vp, BF16, 128, 256)
    assert _call_step(f, _t(f, A, F32, 64, 256), _t(f, B, F32, 64, 128), _t(f, C, F32, 128, 256), mb, vb) == -3
    assert _call_step(f, X, dY, W, _t(f, Mp, BF16, 128, 256, ld=260), vb) == -4  # bf16 moment rows of 8
    assert _call_step(f, X, dY, W, mb, vb, step=1 << 31) == -6                   # step < 2^31
    assert _call_step(f, X, dY, W, _t(f, Mp, I8, 128, 256, scale=S1), v) == -3  # mixed state formats
    assert _call_step(f, X, dY, _t(f, C, F32, 128, 256), m, v) == -3      # W dtype differs from X
    assert _call_step(f, _t(f, A + 2, BF16, 64, 256), dY, W, m, v) == -4  # misaligned pointer
    assert _call_step(f, X, dY, W, m, v, step=0) == -6
    assert _call_step(f, X, dY, W, m, v, opt=9) == -6
    assert _call_step(f, X, dY, W, m, v, hyper={"beta2": 1.0}) == -6
    assert _call_step(f, X, dY, W, m, v, hyper={"lr": float("nan")}) == -6
    assert _call_step(f, X, dY, W, _t(f, C, F32, 128, 256), v) == -8      # m aliases W
    assert _call_step(f, X, dY, W, m, _t(f, A, F32, 128, 256)) == -8      # v aliases X
    q8m = _t(f, Mp, I8, 128, 256, scale=S1)
    q8v = _t(f, Vp, U8, 128, 256, scale=S2)
    assert _call_step(f, X, dY, W, _t(f, Mp, I8, 128, 256), q8v) == -1    # missing scales
    Xf = _t(f, A, F32, 64, 256)
    dYf = _t(f, B, F32, 64, 128)
    Wf = _t(f, C, F32, 128, 256)
    assert _call_step(f, Xf, dYf, Wf, q8m, q8v) == -3                    # INT8 states need bf16 io
    Xr = _t(f, A, BF16, 64, 264)
    Wr = _t(f, C, BF16, 128, 264)
    assert _call_step(f, Xr, dY, Wr, _t(f, Mp, I8, 128, 264, ld=272, scale=S1),
                      _t(f, Vp, U8, 128, 264, ld=272, scale=S2)) == -5    # INT8 needs in % 64 == 0
    # sgd needs no states at all: missing m/v is not an error there (stops before launch only via
    # another error, here an alignment error on X)
    assert _call_step(f, _t(f, A + 8, BF16, 64, 256), dY, W, None, None, opt="sgd") == -4
    r = lambda x: ctypes.byref(x)  # noqa: E731
    lib = f.lib()
    assert lib.forge_linear_dgrad(r(dY), r(W), r(_t(f, A, BF16, 64, 200)), None) == -2
    assert lib.forge_linear_dgrad(r(dY), r(W), r(_t(f, A, F32, 64, 256)), None) == -3
    assert lib.forge_linear_dgrad(r(dY), r(W), r(_t(f, C, BF16, 64, 256)), None) == -8
    assert lib.forge_linear_wgrad(r(X), r(dY), ctypes.c_void_p(0x80000004), 256, None) == -4
    assert lib.forge_linear_wgrad(r(X), r(dY), ctypes.c_void_p(0x80000000), 255, None) == -2
    h = f.make_hyper("adamw")
    assert lib.forge_optimizer_step(ctypes.c_void_p(0x80000000), 256, r(W), r(m), r(v), 0, ctypes.byref(h), 0, 0,
                                    None) == -6
    assert lib.forge_optimizer_step(None, 256, r(W), r(m), r(v), 0, ctypes.byref(h), 1, 0, None) == -1
    assert E.STATUS[-7] == "FORGE_ERR_HIP"
    # the single-call unfused baseline validates its workspace like the other arguments
    WS = 0x7A000000

    def unfused(ws, ld, W_=W, m_=m, v_=v):
        return lib.forge_linear_wgrad_unfused(r(X), r(dY), r(W_), r(m_), r(v_), 0, ctypes.byref(h), 1, 0,
                                              ctypes.c_void_p(ws) if ws else None, ld, None)
    assert unfused(0, 256) == -1                      # no workspace
    assert unfused(WS + 4, 256) == -4                 # misaligned
    assert unfused(WS, 252) == -2                     # ld_ws < in
    assert unfused(WS, 258) == -4                     # ld_ws not a multiple of 4
    assert unfused(C + 64, 256) == -8                 # workspace overlaps W
    assert unfused(Mp, 256) == -8                     # workspace overlaps m
    assert unfused(A, 256) == -8                      # workspace overlaps X
    assert unfused(WS, 256, m_=_t(f, C, F32, 128, 256)) == -8   # m overlaps W (checked as in the fused step)


@cpu_only
def test_alias_checks_cover_scales(f):
    """Block scales of INT8 states and the one-float scales of FP8 inputs take part in the
    overlap check: against each other, against every tensor's data, and their own data."""
    BF16, I8, U8, E4M3, E5M2, F32 = 1, 2, 3, 4, 5, 0
    A, B, C, Mp, Vp = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
    S1, S2 = 0x60000000, 0x70000000          # scales: 128 rows x 4 blocks x 4 bytes = 2 KiB each
    X = _t(f, A, BF16, 64, 256)
    dY = _t(f, B, BF16, 64, 128)
    W = _t(f, C, BF16, 128, 256)
    ok_m, ok_v = _t(f, Mp, I8, 128, 256, scale=S1), _t(f, Vp, U8, 128, 256, scale=S2)
    # m's scales overlap v's scales
    assert _call_step(f, X, dY, W, ok_m, _t(f, Vp, U8, 128, 256, scale=S1 + 1024)) == -8
    # a scale array overlaps an input (X), W, or the other moment's codes
    assert _call_step(f, X, dY, W, _t(f, Mp, I8, 128, 256, scale=A + 64), ok_v) == -8
    assert _call_step(f, X, dY, W, ok_m, _t(f, Vp, U8, 128, 256, scale=C + 4096)) == -8
    assert _call_step(f, X, dY, W, ok_m, _t(f, Vp, U8, 128, 256, scale=Mp + 128)) == -8
    # a moment's own codes overlap its own scales
    assert _call_step(f, X, dY, W, _t(f, Mp, I8, 128, 256, scale=Mp + 256), ok_v) == -8
    # an FP8 input's scale lies inside W, or inside a state's block scales
    m32, v32 = _t(f, Mp, F32, 128, 256), _t(f, Vp, F32, 128, 256)
    Xq = _t(f, A, E4M3, 64, 256, scale=C + 16)
    dYq = _t(f, B, E5M2, 64, 128, scale=S2)
    assert _call_step(f, Xq, dYq, W, m32, v32) == -8
    Xq = _t(f, A, E4M3, 64, 256, scale=S1 + 8)
    assert _call_step(f, Xq, _t(f, B, E5M2, 64, 128, scale=0x7F000000), W, ok_m, ok_v) == -8


@cpu_only
def test_fp8_validation_errors(f):
    """FP8 inputs: X E4M3, dY E4M3 or E5M2, each with a one-float device scale, bf16 W, fp32 moments."""
    F32, BF16, I8, U8, E4M3, E5M2 = 0, 1, 2, 3, 4, 5
    A, B, C, Mp, Vp = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
    SX, SD, S1, S2 = 0x60000000, 0x60000004, 0x70000000, 0x78000000
    X = _t(f, A, E4M3, 64, 256, scale=SX)
    dY = _t(f, B, E5M2, 64, 128, scale=SD)
    W = _t(f, C, BF16, 128, 256)
    m = _t(f, Mp, F32, 128, 256)
    v = _t(f, Vp, F32, 128, 256)
    assert _call_step(f, _t(f, A, E4M3, 64, 256), dY, W, m, v) == -1            # X without its scale
    assert _call_step(f, X, _t(f, B, E5M2, 64, 128), W, m, v) == -1             # dY without its scale
    assert _call_step(f, _t(f, A, E5M2, 64, 256, scale=SX), dY, W, m, v) == -3  # X must be E4M3
    assert _call_step(f, X, dY, _t(f, C, F32, 128, 256), m, v) == -3            # W must be bf16
    assert _call_step(f, X, _t(f, B, BF16, 64, 128), W, m, v) == -3             # mixed FP8 / bf16 inputs
    assert _call_step(f, _t(f, A, E4M3, 64, 264, scale=SX), dY, _t(f, C, BF16, 128, 264), m, v) == -4  # cols % 16
    assert _call_step(f, _t(f, A, E4M3, 64, 256, ld=264, scale=SX), dY, W, m, v) == -4  # ld % 16
    assert _call_step(f, _t(f, A + 8, E4M3, 64, 256, scale=SX), dY, W, m, v) == -4      # 16-byte base
    assert _call_step(f, _t(f, A, E4M3, 64, 256, scale=SX + 2), dY, W, m, v) == -4      # float scale alignment
    assert _call_step(f, X, _t(f, B, E5M2, 63, 128, scale=SD), W, m, v) == -2   # T mismatch
    assert _call_step(f, X, dY, W, _t(f, Mp, I8, 128, 256),
                      _t(f, Vp, U8, 128, 256, scale=S2)) == -1                   # INT8 m with FP8: needs its scales
    r = lambda x: ctypes.byref(x)  # noqa: E731
    lib = f.lib()
    assert lib.forge_linear_dgrad(r(_t(f, B, E4M3, 64, 128, scale=SD)), r(W), r(_t(f, A, BF16, 64, 256)),
                                  None) == -5                                    # no FP8 dgrad
    assert lib.forge_linear_wgrad(r(_t(f, A, E4M3, 64, 256)), r(dY), ctypes.c_void_p(0x80000000), 256,
                                  None) == -1
    assert lib.forge_linear_wgrad(r(X), r(_t(f, B, E5M2, 64, 120, scale=SD)), ctypes.c_void_p(0x80000000), 256,
                                  None) == -4


def test_step_scalars_errors(f):
    s = f.forge.ForgeScalars()
    h = f.make_hyper("adamw")
    lib = f.lib()
    assert lib.forge_step_scalars(0, ctypes.byref(h), 0, ctypes.byref(s)) == -6
    assert lib.forge_step_scalars(0, None, 1, ctypes.byref(s)) == -1
    assert lib.forge_step_scalars(0, ctypes.byref(h), 1, None) == -1
    with pytest.raises(f.ForgeError):
        f.step_scalars("adamw", {"eps": -1.0}, 1)


# ---------------------------------------------------------------- dynamic 8-bit moment code
def test_dyn_table_matches_oracle(f):
    """The library's constexpr tables equal the oracle's code values bit for bit."""
    from oracle import q8
    for k in range(256):
        val = np.float32(f.dyn_value(False, k))
        assert val.view(np.uint32) == q8.DYN_UNSIGNED[k].view(np.uint32), k
        ref = -q8.DYN_SIGNED[k & 0x7F] if k & 0x80 else q8.DYN_SIGNED[k]
        assert np.float32(f.dyn_value(True, k)) == np.float32(ref), k
    assert math.isnan(f.dyn_value(True, 256)) and math.isnan(f.dyn_value(False, -1))


def test_dyn_encode_matches_oracle(f):
    """The library's encoder (the kernels' code, host build) picks the oracle's code for
    random normalised values, for every code value and for the float32 neighbours of
    every midpoint between codes (the decision boundaries)."""
    from oracle import q8
    rng = np.random.default_rng(11)
    for signed, table in ((True, q8.DYN_SIGNED), (False, q8.DYN_UNSIGNED)):
        t64 = table.astype(np.float64)
        mids = ((t64[:-1] + t64[1:]) * 0.5).astype(np.float32)
        ys = [table, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(2)),
              rng.uniform(0, 1, 2000).astype(np.float32), (10.0 ** rng.uniform(-9, 0, 2000)).astype(np.float32)]
        y = np.clip(np.concatenate(ys), 0, 1).astype(np.float32)
        if signed:
            y = np.concatenate([y, -y[: y.size // 2]])
        x = np.zeros((y.size, 64))
        x[:, 0] = 1.0
        x[:, 1] = y
        q, _ = (q8.quant_dyn_signed if signed else q8.quant_dyn_unsigned)(x)
        got = np.array([f.dyn_encode(signed, float(v)) for v in y])
        np.testing.assert_array_equal(got, q[:, 1].astype(np.int64))


@cpu_only
def test_dyn_state_validation(f):
    F32, BF16, I8, U8, E4M3, I8D, U8D = 0, 1, 2, 3, 4, 6, 7
    A, B, C, Mp, Vp, S1, S2 = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x60000000, 0x70000000
    X, dY, W = _t(f, A, BF16, 64, 256), _t(f, B, BF16, 64, 128), _t(f, C, BF16, 128, 256)
    dm, dv = _t(f, Mp, I8D, 128, 256, scale=S1), _t(f, Vp, U8D, 128, 256, scale=S2)
    assert _call_step(f, X, dY, W, dm, _t(f, Vp, U8, 128, 256, scale=S2)) == -3    # linear and dynamic mixed
    assert _call_step(f, X, dY, W, _t(f, Mp, U8D, 128, 256, scale=S1), dv) == -3    # m must be the signed code
    assert _call_step(f, X, dY, W, _t(f, Mp, I8D, 128, 256), dv) == -1             # missing scales
    assert _call_step(f, _t(f, A, F32, 64, 256), _t(f, B, F32, 64, 128), _t(f, C, F32, 128, 256), dm, dv) == -3
    Xr, Wr = _t(f, A, BF16, 64, 264), _t(f, C, BF16, 128, 264)
    assert _call_step(f, Xr, dY, Wr, _t(f, Mp, I8D, 128, 264, ld=272, scale=S1),
                      _t(f, Vp, U8D, 128, 264, ld=272, scale=S2)) == -5             # in % 64 == 0
    one = 0x78000000
    X8 = _t(f, A, E4M3, 64, 256, scale=one)
    dY8 = _t(f, B, E4M3, 64, 128, scale=one + 256)
    assert _call_step(f, X8, dY8, W, dm, _t(f, Vp, U8, 128, 256, scale=S2)) == -3   # mixed codes, FP8 inputs
    assert _call_step(f, X8, dY8, W, _t(f, Mp, I8D, 128, 256), dv) == -1             # scales, FP8 inputs


def test_dyn_fast_encoder_exhaustive(tmp_path):
    """The kernels' dynamic-code encoder (guess + one-step check) equals the binary
    search over the midpoints for every float in [0, 1] (host build of the same code;
    the guess uses only IEEE float operations, so the device computes the same)."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "dyn_exhaustive")
    src = os.path.join(ROOT, "tests", "dyn_encoder_exhaustive.cpp")
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-pthread", src, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("0 mismatches")


@pytest.mark.parametrize("psi", [4e-3, 0.0, 0.5])
def test_nadam_scalars_at_large_steps(f, psi):
    """NAdam's momentum product prod_{k<=t} mu_k, computed by the library in constant
    time, matches the plain product of the oracle's mu_k up to float rounding of the
    kernel arguments, from step 1 to 10^5; a call at step 10^9 stays cheap."""
    import time
    hp = dict(optim.hyper("nadam"), momentum_decay=psi)
    b1, lr = hp["beta1"], hp["lr"]
    prod = 1.0
    marks = {1, 2, 7, 100, 5000, 100000}
    for t in range(1, 100001):
        prod *= optim.nadam_mu(b1, psi, t)
        if t in marks:
            mu_t, mu_n = optim.nadam_mu(b1, psi, t), optim.nadam_mu(b1, psi, t + 1)
            s = f.step_scalars("nadam", dict(momentum_decay=psi), t)
            np.testing.assert_allclose(s["c_g"], lr * (1 - mu_t) / (1 - prod), rtol=2e-6)
            np.testing.assert_allclose(s["c_m"], lr * mu_n / (1 - prod * mu_n), rtol=2e-6)
    c0 = time.perf_counter()
    s = f.step_scalars("nadam", dict(momentum_decay=psi), 10 ** 9)
    assert time.perf_counter() - c0 < 0.05
    mu_inf = b1 * (1 - 0.5 * 0.96 ** (psi * 10 ** 9))
    np.testing.assert_allclose(s["c_m"], lr * mu_inf, rtol=2e-6)  # the product has vanished


def test_nadam_negative_momentum_decay_rejected(f):
    with pytest.raises(f.ForgeError):
        f.step_scalars("nadam", dict(momentum_decay=-1e-3), 1)


@cpu_only
def test_mfma_peak_validation(f):
    lib = f.lib()
    assert lib.forge_mfma_peak(None, 1, 1, 1.0, 1.0, None) == -1
    assert lib.forge_mfma_peak(ctypes.c_void_p(0x10000000), 0, 1, 1.0, 1.0, None) == -5
    assert lib.forge_mfma_peak(ctypes.c_void_p(0x10000000), 1, 0, 1.0, 1.0, None) == -5
    assert lib.forge_mfma_peak(ctypes.c_void_p(0x10000002), 1, 1, 1.0, 1.0, None) == -4
    # 2 flops x 32x32x16 per MFMA, 8 MFMAs per iteration and wave, 4 waves per workgroup
    assert lib.forge_mfma_peak_flops(3, 5) == 2 * 32 * 32 * 16 * 8 * 5 * 4 * 3


def test_bench_refuses_more_than_one_gpu():
    # the measurement covers one GPU; asking for more exits with a message before any GPU work
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_bench_training_workload_rejects_empty_model():
    # the training-step workload checks its block count before any GPU work
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "llama8b_mlp_train_8192",
                        "--blocks", "0"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--blocks" in r.stderr


def _call_group(f, X, dYs, Ws, ms, vs, n=None, opt="adamw", seeds=True):
    h = f.make_hyper(opt)
    k = len(Ws)
    T = f.forge.ForgeTensor
    arr = lambda ts: None if ts is None else (T * k)(*ts)  # noqa: E731
    sd = (ctypes.c_uint64 * k)(*range(k)) if seeds else None
    return f.lib().forge_linear_wgrad_step_group(ctypes.byref(X), k if n is None else n, arr(dYs), arr(Ws), arr(ms),
                                                 arr(vs), f.forge.OPT_ID[opt], ctypes.byref(h), 1, sd, None)


@cpu_only
def test_group_validation(f):
    """The grouped step checks every layer as the single-layer step does, plus the group's own
    rules (1..FORGE_MAX_GROUP layers, one operand format and one moment format, no fp32
    layers, no overlap between layers), all before a launch."""
    F32, BF16, I8, U8, E4M3, E5M2 = 0, 1, 2, 3, 4, 5
    A, B0, B1, C0, C1 = 0x10000000, 0x20000000, 0x21000000, 0x30000000, 0x31000000
    M0, V0, M1, V1, S = 0x40000000, 0x41000000, 0x50000000, 0x51000000, 0x60000000
    X = _t(f, A, BF16, 64, 256)
    dYs = [_t(f, B0, BF16, 64, 128), _t(f, B1, BF16, 64, 64)]
    Ws = [_t(f, C0, BF16, 128, 256), _t(f, C1, BF16, 64, 256)]
    ms = [_t(f, M0, F32, 128, 256), _t(f, M1, F32, 64, 256)]
    vs = [_t(f, V0, F32, 128, 256), _t(f, V1, F32, 64, 256)]
    assert _call_group(f, X, dYs, Ws, ms, vs, n=0) == -2                      # no layer
    assert _call_group(f, X, dYs, Ws, ms, vs, n=f.MAX_GROUP + 1) == -2        # more than the maximum
    assert _call_group(f, X, dYs, Ws, ms, vs, seeds=False) == -1              # no seeds
    assert _call_group(f, X, dYs, [Ws[0], _t(f, C1, BF16, 64, 128)], ms, vs) == -2      # in differs from X's
    assert _call_group(f, X, dYs, Ws, None, vs) == -1                         # AdamW needs m
    assert _call_group(f, X, dYs, [Ws[0], _t(f, C0 + 512, BF16, 64, 256)], ms, vs) == -8  # W of one layer in another's
    assert _call_group(f, X, dYs, Ws, [ms[0], _t(f, V0, F32, 64, 256)], vs) == -8          # m of one layer on v of another
    assert _call_group(f, X, dYs, Ws, [ms[0], _t(f, B1, F32, 64, 256)], vs) == -8          # an output on another layer's dY
    q8 = [_t(f, M1, I8, 64, 256, scale=S), _t(f, V1, U8, 64, 256, scale=S + 4096)]
    assert _call_group(f, X, dYs, Ws, [ms[0], q8[0]], [vs[0], q8[1]]) == -3   # moment formats differ
    Xf = _t(f, A, F32, 64, 256)
    assert _call_group(f, Xf, [_t(f, B0, F32, 64, 128), _t(f, B1, F32, 64, 64)],
                       [_t(f, C0, F32, 128, 256), _t(f, C1, F32, 64, 256)], ms, vs) == -5  # fp32 layers
    Xq = _t(f, A, E4M3, 64, 256, scale=S + 8192)
    assert _call_group(f, Xq, [_t(f, B0, E4M3, 64, 128, scale=S + 8196), _t(f, B1, E5M2, 64, 64, scale=S + 8200)],
                       Ws, ms, vs) == -3                                      # FP8 dY in two formats
    assert _call_group(f, Xq, [_t(f, B0, E4M3, 64, 128, scale=S + 8196), _t(f, B1, BF16, 64, 64)],
                       Ws, ms, vs) == -3                                      # FP8 and bf16 gradients
    assert _call_group(f, Xq, [_t(f, B0, E4M3, 64, 128, scale=S + 8196), _t(f, B1, E4M3, 64, 64)],
                       Ws, ms, vs) == -1                                      # an FP8 dY without its scale


@cpu_only
def test_empty_layer_needs_no_pointers(f):
    # a layer with no weights is a valid no-op: its W and moments may have NULL data (nothing
    # is read, written or launched), alone or as a member of a group
    BF16, F32 = 1, 0
    X = _t(f, 0x10000000, BF16, 64, 256)
    dY = _t(f, 0x20000000, BF16, 64, 0)
    W = _t(f, None, BF16, 0, 256)
    m, v = _t(f, None, F32, 0, 256), _t(f, None, F32, 0, 256)
    assert _call_step(f, X, dY, W, m, v) == 0
    assert _call_group(f, X, [dY], [W], [m], [v]) == 0
    # a layer with weights still needs its moments
    assert _call_step(f, X, _t(f, 0x20000000, BF16, 64, 128), _t(f, 0x30000000, BF16, 128, 256),
                      _t(f, None, F32, 128, 256), v) == -1


def test_grouped_linear_rejects_layers_that_cannot_share_a_launch(f):
    # the check runs on the host before any kernel: layers of a group must agree in
    # optimizer, hyper-parameters, moment format, schedule and step count
    import torch

    from optimizer_gemm_amd.nn import ForgeLinear, grouped_linear
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    a = ForgeLinear(64, 32, device="cpu", seed=1)
    for other in (ForgeLinear(64, 32, device="cpu", seed=2, opt="lion"),
                  ForgeLinear(64, 16, device="cpu", seed=3, hyper={"lr": 5e-4}),
                  ForgeLinear(64, 16, device="cpu", seed=4, states="bf16"),
                  ForgeLinear(64, 16, device="cpu", seed=5, fused=False)):
        with pytest.raises(ValueError):
            grouped_linear([a, other], x)
    b = ForgeLinear(64, 16, device="cpu", seed=6)
    b._step_count = 1
    with pytest.raises(ValueError):
        grouped_linear([a, b], x)
    with pytest.raises(ValueError):
        grouped_linear([a] * (f.MAX_GROUP + 1), x)
