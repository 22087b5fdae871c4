"""GPU parity of the fused step, dgrad and the unfused baseline against the oracle.

Every case draws seeded inputs (synth), runs the HIP path through the C ABI, and
checks each step teacher-forced: the oracle starts each step from the GPU's own
previous W and moments, so per-step tolerances apply (see tests/_parity.py).
Sizes here are small enough for the full float64 oracle, yet span several
tiles with ragged tails in every dimension.
"""
import numpy as np
import pytest
import torch

from oracle import gemm, optim, q8, step
from synth import LayerSpec, draw_layer_batch, draw_layer_init, f32_from_bf16_bits
from tests import _parity as P

pytestmark = pytest.mark.gpu

def _forge():
    import optimizer_gemm_amd as f
    return f


def _gpu_hyper(hp, sr=True):
    d = dict(hp)
    d["nesterov"] = int(bool(d["nesterov"]))
    d["stochastic_round"] = int(sr)
    return d


def run_case(spec, opt, steps, config=90, layer=0, state="f32", sr=True, rows=None, hp_over=None,
             seed=None, label=""):
    f = _forge()
    print(f"[case] {label} opt={opt} spec={spec} state={state} sr={sr} steps={steps}", flush=True)
    io = spec.io
    hp = optim.hyper(opt, **(hp_over or {}))
    seed = (0x5EED0000 + config) ^ layer if seed is None else seed
    W0 = draw_layer_init(config, layer, spec)
    Wd = P.dev_bf16(W0) if io == "bf16" else P.dev(W0)
    m, v, ms, vs = f.new_states(Wd, opt, state)
    sel = np.arange(spec.out) if rows is None else np.asarray(rows)
    for t in range(1, steps + 1):
        X, dY = draw_layer_batch(config, layer, t, spec)
        Xd = P.dev_bf16(X) if io == "bf16" else P.dev(X)
        dYd = P.dev_bf16(dY) if io == "bf16" else P.dev(dY)
        before = P.snapshot((Wd, m, v, ms, vs), sel)
        f.wgrad_step(Xd, dYd, Wd, m, v, opt, _gpu_hyper(hp, sr), t, seed, ms, vs, code=P.state_code(state))
        torch.cuda.synchronize()
        after = P.snapshot((Wd, m, v, ms, vs), sel)
        P.verify_step(opt, X, dY, before, after, hp, t, seed, io, state, sr, sel)
    return Wd, m, v


# ---------------------------------------------------------------- fp32 path
def test_fp32_256_adamw_three_steps():
    run_case(LayerSpec("linear", 256, 256, 512, io="f32", dy_std=1e-2), "adamw", 3, config=0, sr=False,
             label="fp32 256x256 T512")


@pytest.mark.parametrize("opt", optim.OPTIMIZERS)
def test_fp32_ragged_all_optimizers(opt):
    over = {} if opt in ("adamw", "lion") else dict(weight_decay=0.01)
    run_case(LayerSpec("r", 72, 100, 70, io="f32", dy_std=1e-2), opt, 3, config=91, hp_over=over, sr=False,
             label="fp32 ragged")


# ---------------------------------------------------------------- bf16 path
@pytest.mark.parametrize("opt", optim.OPTIMIZERS)
def test_bf16_ragged_all_optimizers_sr(opt):
    # 200 = 128 + 72 rows, 328 = 2*128 + 72 columns, 130 = 2*64 + 2 tokens
    run_case(LayerSpec("r", 200, 328, 130), opt, 3, config=92, label="bf16 ragged")


def test_bf16_nesterov_and_dampening():
    run_case(LayerSpec("r", 136, 264, 96), "sgd_momentum", 3, config=93,
             hp_over=dict(nesterov=True, weight_decay=0.02), label="nesterov")
    run_case(LayerSpec("r", 136, 264, 96), "sgd_momentum", 3, config=93, layer=1,
             hp_over=dict(dampening=0.25), label="dampening")


def test_bf16_round_to_nearest_mode():
    run_case(LayerSpec("r", 256, 384, 256), "adamw", 2, config=94, sr=False, label="bf16 rne")


def test_bf16_several_tiles():
    run_case(LayerSpec("m", 512, 640, 1000), "adamw", 2, config=95, label="bf16 512x640 T1000")


def test_radam_crosses_rectification():
    run_case(LayerSpec("r", 128, 128, 64), "radam", 7, config=96, label="radam 7 steps")


def test_empty_tokens_zero_gradient():
    # T == 0: dW = 0, the optimizer still applies decay/momentum
    run_case(LayerSpec("e", 128, 256, 0), "adamw", 2, config=97, label="T=0")
    run_case(LayerSpec("e", 64, 64, 0, io="f32"), "sgd_momentum", 2, config=97, sr=False, label="T=0 fp32")


# ---------------------------------------------------------------- INT8 states
@pytest.mark.parametrize("opt", ["adamw", "lion", "rmsprop", "sgd_momentum", "nadam"])
def test_q8_states(opt):
    run_case(LayerSpec("q", 136, 320, 200, outlier_frac=0.01), opt, 3, config=98, state="q8", label="q8")


@pytest.mark.parametrize("opt", ["adamw", "lion", "rmsprop", "sgd_momentum", "nadam", "radam", "adagrad"])
def test_q8_dynamic_code_states(opt):
    run_case(LayerSpec("q", 136, 320, 200, outlier_frac=0.01), opt, 3, config=98, layer=1, state="q8dyn",
             label="q8 dynamic code")


# ---------------------------------------------------------------- bfloat16 states
@pytest.mark.parametrize("opt", optim.OPTIMIZERS)
def test_bf16_states_all_optimizers_sr(opt):
    run_case(LayerSpec("r", 200, 328, 130), opt, 3, config=99, state="bf16", label="bf16 states")


def test_bf16_states_round_to_nearest():
    run_case(LayerSpec("r", 136, 264, 96), "adamw", 2, config=99, layer=1, state="bf16", sr=False,
             label="bf16 states rne")


# ---------------------------------------------------------------- tile configurations
def _tile_config_shapes():
    """(rows, cols) of C = (in, out) for wgrad or (in, T) for dgrad that select each
    tile configuration of the launcher on this device: 256x256 tiles when there are
    at least as many as compute units, else 128x128 tiles when there are at least two
    per compute unit, else 128x128 tiles with the in-workgroup split-K, or 64x128 split-K
    tiles (tiny) when those fit in one round and the 128x128 ones would leave compute
    units idle.
    The band_* shapes (256 compute units) leave a last round of 256x256 tiles at most
    half full, so the launcher runs the whole rounds over a band of tile columns or rows
    and the rest as a second launch: band_n (column band, ragged 256x128 rest), band_m
    (row band, ragged 256x128 rest), band_full (a rest of exactly one round of 256x128
    tiles) and band_small (a rest too large for one round of 256x128 tiles, so 128x128)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    big = (4096, 256 * -(-cus // 16))
    small = (4096, 128 * -(-cus // 16))
    split = (2560, 1280)
    tiny = (4096, 128)
    cdiv = lambda a, b: -(-a // b)
    tiles = lambda mn, t, tn=None: cdiv(mn[0], t) * cdiv(mn[1], tn or t)
    assert tiles(big, 256) >= cus
    assert 2 * tiles(small, 256) <= cus and tiles(small, 128) >= 2 * cus
    assert 2 * tiles(split, 256) <= cus and tiles(split, 128) < 2 * cus and tiles(split, 64, 128) > cus
    assert 2 * tiles(tiny, 256) <= cus and tiles(tiny, 128) < tiles(tiny, 64, 128) <= cus
    shapes = {"big": big, "small": small, "split": split, "tiny": tiny}
    if cus == 256:
        shapes.update(band_n=(4096, 4416), band_m=(4416, 4096), band_full=(4096, 6144), band_small=(5120, 4864))
        for k in ("band_n", "band_m", "band_full", "band_small"):
            assert tiles(shapes[k], 256) > cus and 2 * (tiles(shapes[k], 256) % cus) <= cus
    return shapes


def _shape(cfg):
    sh = _tile_config_shapes()
    if cfg not in sh:
        pytest.skip(f"{cfg}: shapes are laid out for 256 compute units")
    return sh[cfg]


CONFIGS = ["big", "small", "split", "tiny", "band_n", "band_m", "band_full", "band_small"]


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("state", ["f32", "q8", "q8dyn", "bf16"])
def test_each_tile_configuration_fused(cfg, state):
    n_in, n_out = _shape(cfg)
    rows = np.unique(np.concatenate([np.arange(0, n_out, max(1, n_out // 96)), [n_out - 1]]))
    run_case(LayerSpec("c", n_out, n_in, 72), "adamw", 2, config=88, state=state, rows=rows,
             label=f"tile config {cfg}")


@pytest.mark.parametrize("cfg", CONFIGS)
def test_each_tile_configuration_dgrad(cfg):
    f = _forge()
    n_in, T = _shape(cfg)
    spec = LayerSpec("d", 136, n_in, T)
    print(f"[case] dgrad tile config {cfg}: T={T} out=136 in={n_in}", flush=True)
    W = draw_layer_init(87, 0, spec)
    X, dY = draw_layer_batch(87, 0, 1, spec)
    dX = f.dgrad(P.dev_bf16(dY), P.dev_bf16(W))
    torch.cuda.synchronize()
    ref = gemm.dgrad(f32_from_bf16_bits(dY), f32_from_bf16_bits(W))
    bad, worst = P.dgrad_bf16_ok(P.host_bits(dX), ref)
    assert bad == 0, f"{bad} dX elements beyond one bf16 ulp (worst {worst:.3g})"


@pytest.mark.parametrize("T", [0, 17, 40])
def test_large_tiles_few_token_stages(T):
    # the 256x256 tiles' mainloop with 0, 1 and 2 stages of 32 tokens: the ring's prologue,
    # the reads ahead into stages past the last one and the closing waits
    n_in, n_out = _shape("big")
    rows = np.unique(np.concatenate([np.arange(0, n_out, max(1, n_out // 64)), [n_out - 1]]))
    run_case(LayerSpec("c", n_out, n_in, T), "adamw", 2, config=89, rows=rows, label=f"256x256 tiles, T={T}")


@pytest.mark.parametrize("n_out", [16, 40])
def test_large_tiles_dgrad_few_stages(n_out):
    # dgrad on 256x256 tiles whose reduction (out) spans one or two 32-row stages
    f = _forge()
    n_in, T = _shape("big")
    spec = LayerSpec("d", n_out, n_in, T)
    print(f"[case] dgrad 256x256 tiles: T={T} out={n_out} in={n_in}", flush=True)
    W = draw_layer_init(86, 0, spec)
    X, dY = draw_layer_batch(86, 0, 1, spec)
    dX = f.dgrad(P.dev_bf16(dY), P.dev_bf16(W))
    torch.cuda.synchronize()
    ref = gemm.dgrad(f32_from_bf16_bits(dY), f32_from_bf16_bits(W))
    bad, worst = P.dgrad_bf16_ok(P.host_bits(dX), ref)
    assert bad == 0, f"{bad} dX elements beyond one bf16 ulp (worst {worst:.3g})"


# ---------------------------------------------------------------- dgrad
@pytest.mark.parametrize("shape,io", [((130, 200, 328), "bf16"), ((512, 384, 256), "bf16"),
                                      ((512, 256, 256), "f32"), ((70, 72, 100), "f32")])
def test_dgrad(shape, io):
    f = _forge()
    T, n_out, n_in = shape
    spec = LayerSpec("d", n_out, n_in, T, io=io)
    W = draw_layer_init(99, 0, spec)
    X, dY = draw_layer_batch(99, 0, 1, spec)
    if io == "bf16":
        dX = f.dgrad(P.dev_bf16(dY), P.dev_bf16(W))
        torch.cuda.synchronize()
        ref = gemm.dgrad(f32_from_bf16_bits(dY), f32_from_bf16_bits(W))
        bad, worst = P.dgrad_bf16_ok(P.host_bits(dX), ref)
        assert bad == 0, f"{bad} dX elements beyond one bf16 ulp (worst {worst:.3g})"
    else:
        dX = f.dgrad(P.dev(dY), P.dev(W))
        torch.cuda.synchronize()
        ref = gemm.dgrad(dY, W)
        abs_sum = np.abs(dY.astype(np.float64)) @ np.abs(W.astype(np.float64))
        bad, worst = P.summation_bound_ok(dX.cpu().numpy(), ref, abs_sum, n_out)
        assert bad == 0, f"{bad} fp32 dX elements beyond the summation bound (worst {worst:.3g})"


def test_dgrad_reads_old_weights_before_step():
    # dgrad enqueued before the fused step on the same stream sees the old W
    f = _forge()
    spec = LayerSpec("o", 256, 256, 256)
    W = draw_layer_init(100, 0, spec)
    X, dY = draw_layer_batch(100, 0, 1, spec)
    Wd = P.dev_bf16(W)
    m, v, _, _ = f.new_states(Wd, "sgd")
    dX = f.dgrad(P.dev_bf16(dY), Wd)
    f.wgrad_step(P.dev_bf16(X), P.dev_bf16(dY), Wd, m, v, "sgd", dict(lr=0.5), 1, 1)
    torch.cuda.synchronize()
    ref = gemm.dgrad(f32_from_bf16_bits(dY), f32_from_bf16_bits(W))
    bad, _ = P.dgrad_bf16_ok(P.host_bits(dX), ref)
    assert bad == 0
    assert not np.array_equal(P.host_bits(Wd), W)  # the step did change W afterwards


# ---------------------------------------------------------------- unfused baseline
@pytest.mark.parametrize("opt,state", [("adamw", "f32"), ("lion", "f32"), ("radam", "f32"), ("adamw", "q8"),
                                       ("rmsprop", "q8"), ("adamw", "q8dyn"), ("rmsprop", "q8dyn"),
                                       ("adamw", "bf16"), ("sgd_momentum", "bf16")])
def test_unfused_matches_fused(opt, state):
    f = _forge()
    spec = LayerSpec("u", 200, 320, 300)
    W0 = draw_layer_init(101, 0, spec)
    outs = []
    for fused in (True, False):
        Wd = P.dev_bf16(W0)
        m, v, ms, vs = f.new_states(Wd, opt, state)
        for t in (1, 2):
            X, dY = draw_layer_batch(101, 0, t, spec)
            args = (P.dev_bf16(X), P.dev_bf16(dY), Wd, m, v, opt, None, t, 7, ms, vs)
            if fused:
                f.wgrad_step(*args, code=P.state_code(state))
            else:
                f.wgrad_unfused(*args, code=P.state_code(state))
        torch.cuda.synchronize()
        outs.append([P.host(x) for x in (Wd, m, v, ms, vs) if x is not None])
    for a, b in zip(*outs):
        if a.dtype == np.uint16:
            ok, n, mx = P.bf16_sr_ok(a, b)
            assert ok, (n, mx)
        elif a.dtype in (np.int8, np.uint8) and state == "q8dyn":
            signed = a.dtype == np.int8
            assert P.codes_ok(q8.dyn_rank(a, signed), q8.dyn_rank(b, signed))[0] == 0
        elif a.dtype in (np.int8, np.uint8):
            assert P.codes_ok(a, b)[0] == 0
        else:
            assert P.state_ok(a, b, rel=1e-6)[0] == 0


def test_unfused_dw_matches_oracle():
    f = _forge()
    spec = LayerSpec("u", 200, 328, 130)
    X, dY = draw_layer_batch(102, 0, 1, spec)
    dW = f.wgrad(P.dev_bf16(X), P.dev_bf16(dY))
    torch.cuda.synchronize()
    Xw, dYw = f32_from_bf16_bits(X).astype(np.float64), f32_from_bf16_bits(dY).astype(np.float64)
    ref = gemm.wgrad(Xw, dYw)
    bad, worst = P.summation_bound_ok(dW.cpu().numpy(), ref, np.abs(dYw).T @ np.abs(Xw), spec.T)
    assert bad == 0, (bad, worst)


# ---------------------------------------------------------------- invariants
def test_bitwise_deterministic_and_resumable():
    f = _forge()
    spec = LayerSpec("d", 384, 512, 700)
    W0 = draw_layer_init(103, 0, spec)
    res = []
    for split in (False, True):
        Wd = P.dev_bf16(W0)
        m, v, _, _ = f.new_states(Wd, "adamw")
        for t in (1, 2, 3, 4):
            if split and t == 3:
                # "checkpoint": round-trip the state through host memory, then continue
                Wd = P.dev_bf16(P.host(Wd))
                m = P.dev(P.host(m))
                v = P.dev(P.host(v))
            X, dY = draw_layer_batch(103, 0, t, spec)
            f.wgrad_step(P.dev_bf16(X), P.dev_bf16(dY), Wd, m, v, "adamw", None, t, 11)
        torch.cuda.synchronize()
        res.append((P.host(Wd), P.host(m), P.host(v)))
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_tensor_parallel_shards_equal_unsharded():
    # exactness under TP (§2 distributed compatibility): row shards (column-parallel layers) and
    # column shards (row-parallel layers) of W, each updated from its local gradient only,
    # reproduce the unsharded update bit for bit. Shards are views of one buffer at tile
    # boundaries, so each element sees the same accumulation order; nearest rounding is used
    # because the stochastic-rounding counter is the index within the tensor passed in.
    f = _forge()
    spec = LayerSpec("tp", 256, 512, 256)
    W0 = draw_layer_init(104, 0, spec)
    X, dY = draw_layer_batch(104, 0, 1, spec)
    Xd, dYd = P.dev_bf16(X), P.dev_bf16(dY)
    hp = dict(stochastic_round=0)
    Wn = P.dev_bf16(W0)
    mn, vn, _, _ = f.new_states(Wn, "adamw")
    f.wgrad_step(Xd, dYd, Wn, mn, vn, "adamw", hp, 1, 5)
    Wr = P.dev_bf16(W0)
    mr, vr, _, _ = f.new_states(Wr, "adamw")
    for r0 in (0, 128):  # column-parallel: split out-rows, dY columns
        f.wgrad_step(Xd, dYd[:, r0:r0 + 128], Wr[r0:r0 + 128], mr[r0:r0 + 128], vr[r0:r0 + 128], "adamw", hp, 1, 5)
    Wc = P.dev_bf16(W0)
    mc, vc, _, _ = f.new_states(Wc, "adamw")
    for c0 in (0, 256):  # row-parallel: split in-columns, X columns
        f.wgrad_step(Xd[:, c0:c0 + 256], dYd, Wc[:, c0:c0 + 256], mc[:, c0:c0 + 256], vc[:, c0:c0 + 256],
                     "adamw", hp, 1, 5)
    torch.cuda.synchronize()
    for got in ((Wr, mr, vr), (Wc, mc, vc)):
        for a, b in zip(got, (Wn, mn, vn)):
            assert np.array_equal(P.host(a), P.host(b))


# ---------------------------------------------------------------- MFMA-peak microbenchmark
def test_mfma_peak_probe_exact_and_plausible():
    # every thread's accumulator sum is exactly 2 * iters (A = 1, B = 2^-10), and the
    # measured rate lies between a floor and the data-sheet dense bf16 peak (2.5 PFLOP/s)
    f = _forge()
    pk = f.mfma_peak(iters=2000, reps=3)
    print(f"[mfma peak] {pk}", flush=True)
    assert 300.0 < pk["tflops"] < 2520.0


# ---------------------------------------------------------------- late steps
@pytest.mark.parametrize("opt,over", [("adamw", {}), ("nadam", {}), ("radam", {}), ("adagrad", {"lr_decay": 1e-3})])
def test_step_one_hundred_thousand_from_nonzero_moments(opt, over):
    # one fused step at t = 100000 from seeded non-zero moments: bias corrections near 1,
    # NAdam's momentum product over 10^5 steps, RAdam in its rectified branch, AdaGrad's
    # decayed rate — the host scalars and the kernel against the oracle's own formulas
    f = _forge()
    spec = LayerSpec("late", 136, 264, 96)
    t = 100_000
    print(f"[case] late step t={t} opt={opt}", flush=True)
    W0 = draw_layer_init(96, 0, spec)
    X, dY = draw_layer_batch(96, 0, 1, spec)
    rng = np.random.default_rng(11)
    m0 = (rng.standard_normal(W0.shape) * 1e-4).astype(np.float32)
    v0 = (rng.standard_normal(W0.shape) ** 2 * 1e-8 + 1e-12).astype(np.float32)
    hp = optim.hyper(opt, **over)
    Wd = P.dev_bf16(W0)
    slots = optim.SLOTS[opt]
    m = P.dev(m0) if "m" in slots else None
    v = P.dev(v0) if "v" in slots else None
    sel = np.arange(spec.out)
    before = P.snapshot((Wd, m, v, None, None), sel)
    f.wgrad_step(P.dev_bf16(X), P.dev_bf16(dY), Wd, m, v, opt, _gpu_hyper(hp), t, 0x5EED_1000)
    torch.cuda.synchronize()
    after = P.snapshot((Wd, m, v, None, None), sel)
    P.verify_step(opt, X, dY, before, after, hp, t, 0x5EED_1000, "bf16", "f32", True, sel)


# ---------------------------------------------------------------- a partial round of large tiles
@pytest.mark.parametrize("state", ["f32", "q8", "q8dyn", "bf16"])
def test_partial_round_of_large_tiles(state):
    # 3584 x 4096: 224 tiles of 256x256, more than half of the 256 compute units, so one
    # partial round of large tiles (and not 896 tiles of 128x128 over two rounds)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip("shape laid out for 256 compute units")
    rows = np.unique(np.concatenate([np.arange(0, 3584, 37), [3583]]))
    run_case(LayerSpec("mr", 3584, 4096, 200), "adamw", 2, config=140, rows=rows, state=state,
             label=f"a partial round of 256x256 tiles, {state} moments")


# ---------------------------------------------------------------- smallest shapes, streams
@pytest.mark.parametrize("out,inn,T", [(8, 8, 1), (8, 16, 3), (8, 64, 1), (136, 8, 17), (24, 1032, 1)])
def test_smallest_shapes(out, inn, T):
    # one token, and 8-wide rows (the least a bf16 row of X or dY may have): single partial
    # tiles whose rows, columns and token range are all ragged, fused step and dgrad
    f = _forge()
    spec = LayerSpec("s", out, inn, T)
    run_case(spec, "adamw", 2, config=105, label=f"smallest {out}x{inn} T={T}")
    X, dY = draw_layer_batch(105, 1, 1, spec)
    W = draw_layer_init(105, 1, spec)
    dX = f.dgrad(P.dev_bf16(dY), P.dev_bf16(W))
    torch.cuda.synchronize()
    ref = gemm.dgrad(f32_from_bf16_bits(dY).astype(np.float64), f32_from_bf16_bits(W).astype(np.float64))
    bad, worst = P.dgrad_bf16_ok(P.host_bits(dX), ref)
    assert bad == 0, (bad, worst)


def test_side_stream_matches_default_stream():
    # the kernels run on the stream the caller passes (here a second torch stream, ordered
    # after the inputs' producer by an event): results equal the default-stream run bit for bit
    f = _forge()
    spec = LayerSpec("st", 264, 392, 150)
    print("[case] side stream vs default stream", flush=True)
    W0 = draw_layer_init(106, 0, spec)
    res = []
    for side in (False, True):
        Wd = P.dev_bf16(W0)
        m, v, _, _ = f.new_states(Wd, "adamw")
        s = torch.cuda.Stream() if side else torch.cuda.current_stream()
        for t in (1, 2):
            X, dY = draw_layer_batch(106, 0, t, spec)
            Xd, dYd = P.dev_bf16(X), P.dev_bf16(dY)
            ready = torch.cuda.Event()
            ready.record(torch.cuda.current_stream())
            s.wait_event(ready)
            with torch.cuda.stream(s):
                dX = f.dgrad(dYd, Wd)
                f.wgrad_step(Xd, dYd, Wd, m, v, "adamw", None, t, 13)
            if side:
                # the side stream's tensors outlive their use there
                for tns in (Xd, dYd, dX):
                    tns.record_stream(s)
        s.synchronize()
        torch.cuda.synchronize()
        res.append((P.host(Wd), P.host(m), P.host(v), P.host(dX)))
    for a, b in zip(*res):
        assert np.array_equal(a, b)
