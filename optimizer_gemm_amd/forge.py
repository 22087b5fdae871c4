"""Python binding of libforge.so (ctypes): argument marshalling only.

Every computation runs in the library's HIP kernels. PyTorch provides device
memory and the current HIP stream; tensors are described to the C ABI by data
pointer, dtype, shape and row pitch. There is no fallback: if the library is
not built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FORGE_LIB", os.path.join(_PKG, "_lib", "libforge.so"))

F32, BF16, I8, U8, E4M3, E5M2, I8_DYN, U8_DYN = 0, 1, 2, 3, 4, 5, 6, 7
OPTIMIZERS = ("adamw", "sgd", "sgd_momentum", "lion", "rmsprop", "adagrad", "nadam", "radam")
OPT_ID = {name: k for k, name in enumerate(OPTIMIZERS)}
# slot usage per optimizer: (uses m, uses v)
SLOTS = {"adamw": (1, 1), "sgd": (0, 0), "sgd_momentum": (1, 0), "lion": (1, 0), "rmsprop": (0, 1),
         "adagrad": (0, 1), "nadam": (1, 1), "radam": (1, 1)}

STATUS = {0: "FORGE_OK", -1: "FORGE_ERR_NULL", -2: "FORGE_ERR_SHAPE", -3: "FORGE_ERR_DTYPE",
          -4: "FORGE_ERR_ALIGN", -5: "FORGE_ERR_UNSUPPORTED", -6: "FORGE_ERR_HYPER", -7: "FORGE_ERR_HIP",
          -8: "FORGE_ERR_ALIAS", -9: "FORGE_ERR_SCRATCH"}


class ForgeTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("scale", ctypes.c_void_p)]


class ForgeHyper(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("momentum", ctypes.c_double),
                ("dampening", ctypes.c_double), ("alpha", ctypes.c_double), ("lr_decay", ctypes.c_double),
                ("momentum_decay", ctypes.c_double), ("nesterov", ctypes.c_int32),
                ("stochastic_round", ctypes.c_int32)]


class ForgeScalars(ctypes.Structure):
    _fields_ = [(n, ctypes.c_float) for n in ("lr", "decay", "wd", "b1", "omb1", "b2", "omb2", "step_size",
                                              "inv_sqrt_bc2", "eps", "c_g", "c_m")] + \
               [("flag", ctypes.c_int32), ("opt", ctypes.c_int32)]


class ForgeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_str(status)})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libforge.so not built at {LIB_PATH}; run `python optimizer_gemm_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sigs = {
        "forge_linear_wgrad_step": ([P(ForgeTensor)] * 5 + [ctypes.c_int32, P(ForgeHyper), ctypes.c_int64,
                                                             ctypes.c_uint64, ctypes.c_void_p], ctypes.c_int),
        "forge_linear_wgrad_step_group": ([P(ForgeTensor), ctypes.c_int32] + [P(ForgeTensor)] * 4 +
                                          [ctypes.c_int32, P(ForgeHyper), ctypes.c_int64, P(ctypes.c_uint64),
                                           ctypes.c_void_p], ctypes.c_int),
        "forge_linear_dgrad": ([P(ForgeTensor)] * 3 + [ctypes.c_void_p], ctypes.c_int),
        "forge_linear_wgrad": ([P(ForgeTensor), P(ForgeTensor), ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p],
                               ctypes.c_int),
        "forge_optimizer_step": ([ctypes.c_void_p, ctypes.c_int64] + [P(ForgeTensor)] * 3 +
                                 [ctypes.c_int32, P(ForgeHyper), ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p],
                                 ctypes.c_int),
        "forge_linear_wgrad_unfused": ([P(ForgeTensor)] * 5 + [ctypes.c_int32, P(ForgeHyper), ctypes.c_int64,
                                                                ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64,
                                                                ctypes.c_void_p], ctypes.c_int),
        "forge_linear_wgrad_unfused_noalloc": ([P(ForgeTensor)] * 5 + [ctypes.c_int32, P(ForgeHyper), ctypes.c_int64,
                                                                        ctypes.c_uint64, ctypes.c_void_p], ctypes.c_int),
        "forge_step_scalars": ([ctypes.c_int32, P(ForgeHyper), ctypes.c_int64, P(ForgeScalars)], ctypes.c_int),
        "forge_default_hyper": ([ctypes.c_int32, P(ForgeHyper)], ctypes.c_int),
        "forge_rand16": ([ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32], ctypes.c_uint32),
        "forge_sr_bf16": ([ctypes.c_float, ctypes.c_uint32], ctypes.c_uint16),
        "forge_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "forge_dyn_value": ([ctypes.c_int32, ctypes.c_int32], ctypes.c_float),
        "forge_mfma_peak": ([ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                             ctypes.c_void_p], ctypes.c_int),
        "forge_mfma_peak_flops": ([ctypes.c_int32, ctypes.c_int32], ctypes.c_double),
        "forge_dyn_encode": ([ctypes.c_int32, ctypes.c_float], ctypes.c_int32),
        "forge_version": ([], ctypes.c_int),
    }
    for name, (argt, rest) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = rest
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def status_str(status: int) -> str:
    return _lib.forge_status_str(int(status)).decode()


def version() -> int:
    return _lib.forge_version()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8, torch.uint8: U8,
       torch.float8_e4m3fn: E4M3, torch.float8_e5m2: E5M2}
_FP8 = (torch.float8_e4m3fn, torch.float8_e5m2)


def describe(t: Optional[torch.Tensor], scale: Optional[torch.Tensor] = None, *, device: bool = True,
             code: str = "linear"):
    """forge_tensor for a 2-D row-major tensor (None -> None). int8 / uint8 moments
    hold linear codes (code="linear") or the dynamic 8-bit code (code="dynamic")."""
    if t is None:
        return None
    if code not in ("linear", "dynamic"):
        raise ValueError(f"unknown moment code {code!r}")
    if t.dim() != 2:
        raise ValueError("forge tensors are 2-D")
    if device and not t.is_cuda:
        raise ValueError("forge kernels take device tensors")
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    if t.numel() == 0:
        return ForgeTensor(None, _DT[t.dtype], 0, t.shape[0], t.shape[1], t.shape[1],
                           scale.data_ptr() if scale is not None and scale.numel() else None)
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride(1) == 1)")
    ld = t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))
    if scale is not None:
        if device and not scale.is_cuda:
            raise ValueError("scales must be device tensors")
        if scale.dtype != torch.float32 or not scale.is_contiguous():
            raise ValueError("scales are contiguous float32")
        if t.dtype in _FP8:
            if scale.numel() != 1:
                raise ValueError("an FP8 tensor has one float32 scale")
        elif tuple(scale.shape) != (t.shape[0], t.shape[1] // 64):
            raise ValueError("block scale shape must be [rows, cols/64]")
    elif t.dtype in _FP8:
        raise ValueError("an FP8 tensor needs its float32 scale")
    dt = _DT[t.dtype]
    if code == "dynamic" and dt in (I8, U8):
        dt = I8_DYN if dt == I8 else U8_DYN
    return ForgeTensor(t.data_ptr(), dt, 0, t.shape[0], t.shape[1], ld,
                       scale.data_ptr() if scale is not None else None)


def _ref(x):
    return ctypes.byref(x) if x is not None else None


def default_hyper(opt: str) -> Dict[str, float]:
    h = ForgeHyper()
    st = _lib.forge_default_hyper(OPT_ID[opt], ctypes.byref(h))
    if st:
        raise ForgeError(st, "forge_default_hyper")
    return {n: getattr(h, n) for n, _ in ForgeHyper._fields_}


def make_hyper(opt: str, **over) -> ForgeHyper:
    d = default_hyper(opt)
    for k, v in over.items():
        if k not in d:
            raise KeyError(k)
        d[k] = v
    h = ForgeHyper()
    for n, _ in ForgeHyper._fields_:
        setattr(h, n, int(d[n]) if n in ("nesterov", "stochastic_round") else float(d[n]))
    return h


def _hyper(opt: str, hyper) -> ForgeHyper:
    if isinstance(hyper, ForgeHyper):
        return hyper
    return make_hyper(opt, **(hyper or {}))


def step_scalars(opt: str, hyper=None, step: int = 1) -> Dict[str, float]:
    s = ForgeScalars()
    st = _lib.forge_step_scalars(OPT_ID[opt], ctypes.byref(_hyper(opt, hyper)), int(step), ctypes.byref(s))
    if st:
        raise ForgeError(st, "forge_step_scalars")
    return {n: getattr(s, n) for n, _ in ForgeScalars._fields_}


def rand16(seed: int, step: int, idx: int) -> int:
    return int(_lib.forge_rand16(seed & (2 ** 64 - 1), int(step), int(idx)))


def sr_bf16(x: float, r16: int) -> int:
    return int(_lib.forge_sr_bf16(float(x), int(r16)))


def mfma_peak(n_workgroups: Optional[int] = None, iters: int = 4000, reps: int = 5, stream=None) -> Dict[str, float]:
    """Achieved bf16 MFMA rate of the device (the library's microbenchmark): median
    TFLOP/s over `reps` timed launches on the current stream, after one warm-up. The
    outputs are checked exactly (A = 1, B = 2^-10: every thread writes 2 * iters)."""
    if n_workgroups is None:
        n_workgroups = 3 * torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    out = torch.empty(n_workgroups * 256, dtype=torch.float32, device="cuda")
    st = _stream(stream)
    times = []
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = _lib.forge_mfma_peak(out.data_ptr(), n_workgroups, iters, 1.0, 2.0 ** -10, st)
        e1.record()
        if rc:
            raise ForgeError(rc, "forge_mfma_peak")
        torch.cuda.synchronize()
        if r:
            times.append(e0.elapsed_time(e1))
    if not bool(torch.all(out == 2.0 * iters)):
        raise RuntimeError("forge_mfma_peak: accumulator check failed")
    ms = sorted(times)[len(times) // 2]
    flops = _lib.forge_mfma_peak_flops(n_workgroups, iters)
    return {"tflops": flops / (ms * 1e-3) / 1e12, "ms": ms, "workgroups": n_workgroups, "iters": iters}


def dyn_value(is_signed: bool, code: int) -> float:
    """Value of a dynamic 8-bit moment code (host helper of the library)."""
    return float(_lib.forge_dyn_value(int(bool(is_signed)), int(code)))


def dyn_encode(is_signed: bool, y: float) -> int:
    """The dynamic code the kernels store for a normalised value y (host helper)."""
    return int(_lib.forge_dyn_encode(int(bool(is_signed)), float(y)))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def wgrad_step(X: torch.Tensor, dY: torch.Tensor, W: torch.Tensor, m: Optional[torch.Tensor],
               v: Optional[torch.Tensor], opt: str = "adamw", hyper=None, step: int = 1, seed: int = 0,
               m_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None, stream=None,
               x_scale: Optional[torch.Tensor] = None, dy_scale: Optional[torch.Tensor] = None,
               code: str = "linear") -> None:
    """Fused dW = dY^T X + optimizer step; W, m, v (and scales) updated in place.

    FP8 inputs (X float8_e4m3fn, dY float8_e4m3fn or float8_e5m2) carry their
    dequantisation scales as one-element float32 device tensors x_scale, dy_scale.
    int8 / uint8 moments hold linear codes, or the dynamic 8-bit code with code="dynamic".
    """
    h = _hyper(opt, hyper)
    st = _lib.forge_linear_wgrad_step(_ref(describe(X, x_scale)), _ref(describe(dY, dy_scale)), _ref(describe(W)),
                                      _ref(describe(m, m_scale, code=code)), _ref(describe(v, v_scale, code=code)),
                                      OPT_ID[opt],
                                      ctypes.byref(h), int(step), seed & (2 ** 64 - 1), _stream(stream))
    if st:
        raise ForgeError(st, "forge_linear_wgrad_step")


MAX_GROUP = 4


def wgrad_step_group(X: torch.Tensor, dYs, Ws, ms, vs, opt: str = "adamw", hyper=None, step: int = 1, seeds=(0,),
                     m_scales=None, v_scales=None, stream=None, code: str = "linear",
                     x_scale: Optional[torch.Tensor] = None, dy_scales=None) -> None:
    """Fused steps of the layers that share the input X, in one launch (forge_linear_wgrad_step_group):
    layer l has gradient dYs[l], weights Ws[l], moments ms[l] / vs[l] (lists; None entries, or
    None for the whole list, where the optimizer keeps no such slot) and seed seeds[l]. FP8
    inputs as in wgrad_step: x_scale for X, dy_scales[l] for dYs[l]."""
    n = len(Ws)
    if not (len(dYs) == n and len(seeds) == n) or n < 1 or n > MAX_GROUP:
        raise ValueError(f"a group holds 1..{MAX_GROUP} layers, each with its dY, W and seed")

    def arr(ts, scales=None):
        if ts is None or all(t is None for t in ts):
            return None
        if any(t is None for t in ts):
            raise ValueError("a moment slot is given for some layers of the group and not others")
        sc = scales if scales is not None else [None] * n
        return (ForgeTensor * n)(*[describe(t, s, code=code) for t, s in zip(ts, sc)])

    h = _hyper(opt, hyper)
    dy_a, w_a = arr(dYs, dy_scales), arr(Ws)
    m_a, v_a = arr(ms, m_scales), arr(vs, v_scales)
    seeds_a = (ctypes.c_uint64 * n)(*[s & (2 ** 64 - 1) for s in seeds])
    st = _lib.forge_linear_wgrad_step_group(_ref(describe(X, x_scale)), n, dy_a, w_a, m_a, v_a, OPT_ID[opt],
                                            ctypes.byref(h),
                                            int(step), seeds_a, _stream(stream))
    if st:
        raise ForgeError(st, "forge_linear_wgrad_step_group")


def dgrad(dY: torch.Tensor, W: torch.Tensor, dX: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dX = dY W (from the weights as they are now, i.e. before the step)."""
    if dX is None:
        dX = torch.empty((dY.shape[0], W.shape[1]), dtype=W.dtype, device=W.device)
    st = _lib.forge_linear_dgrad(_ref(describe(dY)), _ref(describe(W)), _ref(describe(dX)), _stream(stream))
    if st:
        raise ForgeError(st, "forge_linear_dgrad")
    return dX


def wgrad(X: torch.Tensor, dY: torch.Tensor, dW: Optional[torch.Tensor] = None, stream=None,
          x_scale: Optional[torch.Tensor] = None, dy_scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Unfused baseline part 1: float32 dW = dY^T X written to device memory (FP8 inputs as in wgrad_step)."""
    if dW is None:
        dW = torch.empty((dY.shape[1], X.shape[1]), dtype=torch.float32, device=X.device)
    if dW.dtype != torch.float32 or dW.dim() != 2 or (dW.shape[1] > 1 and dW.stride(1) != 1) or not dW.is_cuda:
        raise ValueError("dW must be a row-major float32 device tensor")
    st = _lib.forge_linear_wgrad(_ref(describe(X, x_scale)), _ref(describe(dY, dy_scale)), dW.data_ptr(),
                                 dW.stride(0), _stream(stream))
    if st:
        raise ForgeError(st, "forge_linear_wgrad")
    return dW


def optimizer_step(dW: torch.Tensor, W: torch.Tensor, m: Optional[torch.Tensor], v: Optional[torch.Tensor],
                   opt: str = "adamw", hyper=None, step: int = 1, seed: int = 0,
                   m_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                   stream=None, code: str = "linear") -> None:
    """Unfused baseline part 2: element-wise optimizer pass reading the stored dW."""
    if dW.dtype != torch.float32 or not dW.is_cuda or (dW.shape[1] > 1 and dW.stride(1) != 1):
        raise ValueError("dW must be a row-major float32 device tensor")
    h = _hyper(opt, hyper)
    st = _lib.forge_optimizer_step(dW.data_ptr(), dW.stride(0), _ref(describe(W)),
                                   _ref(describe(m, m_scale, code=code)), _ref(describe(v, v_scale, code=code)),
                                   OPT_ID[opt], ctypes.byref(h), int(step),
                                   seed & (2 ** 64 - 1), _stream(stream))
    if st:
        raise ForgeError(st, "forge_optimizer_step")


def _workspace(ws: Optional[torch.Tensor], W: torch.Tensor) -> torch.Tensor:
    if ws is None:
        ws = torch.empty(tuple(W.shape), dtype=torch.float32, device=W.device)
    if ws.dtype != torch.float32 or ws.dim() != 2 or (ws.shape[1] > 1 and ws.stride(1) != 1) or not ws.is_cuda:
        raise ValueError("dW_workspace must be a row-major float32 device tensor")
    return ws


def wgrad_unfused(X, dY, W, m, v, opt="adamw", hyper=None, step=1, seed=0, m_scale=None, v_scale=None,
                  dW_workspace: Optional[torch.Tensor] = None, stream=None, x_scale=None,
                  dy_scale=None, code: str = "linear") -> torch.Tensor:
    """The two-phase baseline in one call (forge_linear_wgrad_unfused): float32 dW into the
    workspace (allocated here if not given), then a separate optimizer pass. Returns dW."""
    ws = _workspace(dW_workspace, W)
    h = _hyper(opt, hyper)
    st = _lib.forge_linear_wgrad_unfused(_ref(describe(X, x_scale)), _ref(describe(dY, dy_scale)), _ref(describe(W)),
                                         _ref(describe(m, m_scale, code=code)), _ref(describe(v, v_scale, code=code)),
                                         OPT_ID[opt], ctypes.byref(h), int(step), seed & (2 ** 64 - 1),
                                         ws.data_ptr() if ws.numel() else None, ws.stride(0), _stream(stream))
    if st:
        raise ForgeError(st, "forge_linear_wgrad_unfused")
    return ws


def wgrad_unfused_noalloc(X, dY, W, m, v, opt="adamw", hyper=None, step=1, seed=0, m_scale=None, v_scale=None,
                          stream=None, x_scale=None, dy_scale=None, code: str = "linear") -> None:
    """The two-phase baseline with dW in the library's static per-GPU scratch
    (forge_linear_wgrad_unfused_noalloc): allocates nothing; out*in <= 2^24."""
    h = _hyper(opt, hyper)
    st = _lib.forge_linear_wgrad_unfused_noalloc(_ref(describe(X, x_scale)), _ref(describe(dY, dy_scale)),
                                                 _ref(describe(W)), _ref(describe(m, m_scale, code=code)),
                                                 _ref(describe(v, v_scale, code=code)), OPT_ID[opt], ctypes.byref(h),
                                                 int(step), seed & (2 ** 64 - 1), _stream(stream))
    if st:
        raise ForgeError(st, "forge_linear_wgrad_unfused_noalloc")


def new_states(W: torch.Tensor, opt: str = "adamw", fmt: str = "f32"):
    """Zero moment slots for `opt` in format f32, bf16, q8 (linear codes) or q8dyn (dynamic
    codes; pass code="dynamic" to the step): returns (m, v, m_scale, v_scale)."""
    use_m, use_v = SLOTS[opt]
    rows, cols = W.shape
    m = v = ms = vs = None
    if fmt == "f32":
        if use_m:
            m = torch.zeros((rows, cols), dtype=torch.float32, device=W.device)
        if use_v:
            v = torch.zeros((rows, cols), dtype=torch.float32, device=W.device)
    elif fmt == "bf16":
        if use_m:
            m = torch.zeros((rows, cols), dtype=torch.bfloat16, device=W.device)
        if use_v:
            v = torch.zeros((rows, cols), dtype=torch.bfloat16, device=W.device)
    elif fmt in ("q8", "q8dyn"):
        if use_m:
            m = torch.zeros((rows, cols), dtype=torch.int8, device=W.device)
            ms = torch.zeros((rows, cols // 64), dtype=torch.float32, device=W.device)
        if use_v:
            v = torch.zeros((rows, cols), dtype=torch.uint8, device=W.device)
            vs = torch.zeros((rows, cols // 64), dtype=torch.float32, device=W.device)
    else:
        raise ValueError(fmt)
    return m, v, ms, vs
