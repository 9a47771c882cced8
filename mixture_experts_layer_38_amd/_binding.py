"""ctypes binding of libmoe_mi355x.so (include/moe.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the layer runs in the library's kernels.
Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_MI355X_DEBUG=1 loads the bounds-checked debug build instead
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x_debug.so" if os.environ.get("MOE_MI355X_DEBUG") == "1"
                        else "libmoe_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_OOM, MOE_ERR_HIP, MOE_ERR_SCRATCH = 0, -1, -2, -3, -4, -5
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_PATH_AUTO, MOE_PATH_GROUPED, MOE_PATH_STREAM = 0, 1, 2
MOE_ACT_QUANT_NONE, MOE_ACT_QUANT_E4M3_1X128 = 0, 1

_DTYPE_CODE = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}
_TORCH_OF = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_FP8_E4M3: torch.uint8}


class MoeParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("dim", "n_routed", "hidden", "shared_hidden", "top_k", "n_group",
                                             "topk_group", "score_fn", "norm_topk")] + \
               [("routed_scaling_factor", ctypes.c_float)] + \
               [(n, ctypes.c_int) for n in ("act_dtype", "weight_dtype", "out_dtype", "add_residual",
                                             "max_tokens", "path", "act_quant", "backward")]


class MoeWeights(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_up_scale", ctypes.c_void_p), ("down_scale", ctypes.c_void_p)]


class MoeWeightGrads(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("down", ctypes.c_void_p)]


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        msg = f"{what}: {status_string(status)} ({status})"
        if hip_error:
            msg += f", HIP error {hip_error}"
        super().__init__(msg)


_lib = None


def load_library() -> ctypes.CDLL:
    """The built HIP library; raises if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_38_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    lib.moe_cfg_create.argtypes = [ctypes.POINTER(MoeParams), ctypes.POINTER(vp)]
    lib.moe_cfg_destroy.argtypes = [vp]
    lib.moe_cfg_workspace_bytes.argtypes = [vp]
    lib.moe_cfg_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_cfg_last_hip_error.argtypes = [vp]
    lib.moe_layer_forward.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.POINTER(MoeWeights),
                                      ctypes.POINTER(MoeWeights), vp, vp, vp]
    lib.moe_router_forward.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp]
    lib.moe_dispatch_forward.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp]
    lib.moe_cfg_set_stage_timing.argtypes = [vp, ctypes.c_int]
    lib.moe_cfg_stage_times.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_bias_update.argtypes = [vp, ctypes.c_int, ctypes.c_float, vp, vp]
    lib.moe_load_stats.argtypes = [vp, ctypes.c_int, vp, vp]
    lib.moe_quantize_e4m3_1x128.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.moe_cfg_set_score_sums.argtypes = [vp, vp]
    lib.moe_debug_status.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.moe_layer_forward_noalloc.argtypes = [ctypes.POINTER(MoeParams), vp, ctypes.c_int, vp, vp,
                                              ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeWeights), vp, vp, vp]
    lib.moe_balance_stats.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.moe_layer_backward.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.POINTER(MoeWeights),
                                       ctypes.POINTER(MoeWeights), vp, vp, vp, ctypes.POINTER(MoeWeightGrads),
                                       ctypes.POINTER(MoeWeightGrads), vp]
    lib.moe_layer_forward_train.argtypes = lib.moe_layer_forward.argtypes
    lib.moe_layer_backward_saved.argtypes = lib.moe_layer_backward.argtypes
    for f in ("moe_cfg_create", "moe_cfg_destroy", "moe_layer_forward", "moe_router_forward",
              "moe_dispatch_forward", "moe_cfg_last_hip_error", "moe_cfg_set_stage_timing",
              "moe_cfg_stage_times", "moe_bias_update", "moe_load_stats", "moe_quantize_e4m3_1x128",
              "moe_layer_backward", "moe_cfg_set_score_sums", "moe_balance_stats",
              "moe_layer_forward_noalloc", "moe_debug_status", "moe_layer_forward_train",
              "moe_layer_backward_saved"):
        getattr(lib, f).restype = ctypes.c_int
    del i32p
    _lib = lib
    return lib


def declared_functions() -> list[str]:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensor(name, t, dtype, shape, device):
    """Raises ValueError unless t is a contiguous tensor of this dtype and
    shape on `device` (a bare device pointer carries none of these)."""
    if not torch.is_tensor(t):
        raise ValueError(f"{name} must be a tensor, got {type(t).__name__}")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_params(*, dim, n_routed, hidden, shared_hidden, top_k, n_group=1, topk_group=1,
                score_fn="softmax", norm_topk=False, routed_scaling_factor=1.0, act="bf16", weight="bf16",
                out="f32", add_residual=True, max_tokens, path="auto", act_quant=False,
                backward=False) -> MoeParams:
    return MoeParams(dim=dim, n_routed=n_routed, hidden=hidden, shared_hidden=shared_hidden, top_k=top_k,
                     n_group=n_group, topk_group=topk_group,
                     score_fn={"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}.get(score_fn, score_fn),
                     norm_topk=int(bool(norm_topk)), routed_scaling_factor=float(routed_scaling_factor),
                     act_dtype=_DTYPE_CODE.get(act, act), weight_dtype=_DTYPE_CODE.get(weight, weight),
                     out_dtype=_DTYPE_CODE.get(out, out), add_residual=int(bool(add_residual)),
                     max_tokens=max_tokens,
                     path={"auto": MOE_PATH_AUTO, "grouped": MOE_PATH_GROUPED, "stream": MOE_PATH_STREAM}.get(path, path),
                     act_quant=int(act_quant), backward=int(bool(backward)))


def create_cfg(params: MoeParams) -> tuple[int, ctypes.c_void_p]:
    """(status, handle) of moe_cfg_create; no exception, for validation tests."""
    h = ctypes.c_void_p()
    st = load_library().moe_cfg_create(ctypes.byref(params), ctypes.byref(h))
    return st, h


def _weights(w) -> MoeWeights | None:
    if w is None:
        return None
    return MoeWeights(w.gate_up.data_ptr(), w.down.data_ptr(),
                      None if getattr(w, "gate_up_scale", None) is None else w.gate_up_scale.data_ptr(),
                      None if getattr(w, "down_scale", None) is None else w.down_scale.data_ptr())


class MoELayer:
    """One cfg (validated parameters + device workspace) of the layer forward."""

    def __init__(self, params: MoeParams):
        self.lib = load_library()
        self.params = params
        st, h = create_cfg(params)
        if st != MOE_OK:
            raise MoEError(st, "moe_cfg_create")
        self.handle = h

    @classmethod
    def from_config(cls, cfg, max_tokens=None, path="auto", **overrides):
        """From an object with the fields of a layer description (T, D, E, H,
        G, kg, K, score_fn, norm, rsf, Hs, act, weight, out, add_residual, and
        optionally act_quant)."""
        kw = dict(dim=cfg.D, n_routed=cfg.E, hidden=cfg.H, shared_hidden=cfg.Hs, top_k=cfg.K, n_group=cfg.G,
                  topk_group=cfg.kg, score_fn=cfg.score_fn, norm_topk=cfg.norm, routed_scaling_factor=cfg.rsf,
                  act=cfg.act, weight=cfg.weight, out=cfg.out, add_residual=cfg.add_residual,
                  max_tokens=cfg.T if max_tokens is None else max_tokens, path=path,
                  act_quant=getattr(cfg, "act_quant", False))
        kw.update(overrides)
        return cls(make_params(**kw))

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            self.lib.moe_cfg_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def workspace_bytes(self) -> int:
        return int(self.lib.moe_cfg_workspace_bytes(self.handle))

    STAGES = ("router", "dispatch", "gate_up_gemm", "down_gemm", "combine")

    def set_stage_timing(self, enable: bool):
        self._check(self.lib.moe_cfg_set_stage_timing(self.handle, int(bool(enable))), "moe_cfg_set_stage_timing")

    def stage_times(self) -> tuple[dict, int]:
        """({stage: summed ms}, timed calls) since the last read; waits for the last call."""
        ms = (ctypes.c_double * len(self.STAGES))()
        calls = ctypes.c_int()
        self._check(self.lib.moe_cfg_stage_times(self.handle, ms, ctypes.byref(calls)), "moe_cfg_stage_times")
        return dict(zip(self.STAGES, list(ms))), calls.value

    def set_score_sums(self, score_sum):
        """moe_cfg_set_score_sums: later forward / router calls also write the
        column sums of the scores into score_sum ([E] fp32 cuda tensor, kept
        alive by the layer); None turns it off."""
        if score_sum is not None:
            _check_tensor("score_sum", score_sum, torch.float32, (self.params.n_routed,), score_sum.device)
            if not score_sum.is_cuda:
                raise ValueError("score_sum must be a cuda tensor")
        self._score_sum = score_sum
        self._check(self.lib.moe_cfg_set_score_sums(self.handle, _ptr(score_sum)), "moe_cfg_set_score_sums")

    def _check(self, st, what):
        if st != MOE_OK:
            raise MoEError(st, what, self.lib.moe_cfg_last_hip_error(self.handle))

    def _check_x(self, x):
        p = self.params
        want = _TORCH_OF[p.act_dtype]
        if (not torch.is_tensor(x) or x.dtype != want or not x.is_cuda or not x.is_contiguous() or x.dim() != 2
                or x.shape[1] != p.dim):
            raise ValueError(f"x must be a contiguous cuda {want} tensor [T, {p.dim}]")

    def _check_router_inputs(self, x, gate_w, sel_bias):
        p = self.params
        _check_tensor("gate_w", gate_w, torch.float32, (p.n_routed, p.dim), x.device)
        if sel_bias is not None:
            _check_tensor("sel_bias", sel_bias, torch.float32, (p.n_routed,), x.device)

    def _check_weights(self, x, experts, shared):
        """Expert and shared weights against the cfg: dtype, shape, device,
        contiguity (the library receives bare pointers and cannot)."""
        p = self.params
        E, D, H, Hs = p.n_routed, p.dim, p.hidden, p.shared_hidden
        wdt = _TORCH_OF[p.weight_dtype]
        fp8 = p.weight_dtype == MOE_FP8_E4M3
        sets = [("experts", experts, (E,), H)]
        if Hs > 0:
            if shared is None:
                raise ValueError("this layer has a shared expert (shared_hidden > 0): pass its weights")
            sets.append(("shared", shared, (), Hs))
        for name, w, lead, h in sets:
            if w is None:
                raise ValueError(f"{name} weights missing")
            _check_tensor(f"{name}.gate_up", w.gate_up, wdt, lead + (2 * h, D), x.device)
            _check_tensor(f"{name}.down", w.down, wdt, lead + (D, h), x.device)
            if fp8:
                _check_tensor(f"{name}.gate_up_scale", getattr(w, "gate_up_scale", None), torch.float32,
                              lead + (2 * h // 128, D // 128), x.device)
                _check_tensor(f"{name}.down_scale", getattr(w, "down_scale", None), torch.float32,
                              lead + (D // 128, h // 128), x.device)

    def forward(self, x, gate_w, sel_bias, experts, shared, out=None, expert_counts=None, stream=None,
                train=False):
        """out [T, D] (out dtype) and, if given, expert_counts [E] int32 are written.
        train=True: the forward of a training step (moe_layer_forward_train; the
        cfg needs backward=True), which also keeps what backward(saved=True)
        reads."""
        p = self.params
        self._check_x(x)
        T = x.shape[0]
        self._check_router_inputs(x, gate_w, sel_bias)
        self._check_weights(x, experts, shared)
        if p.shared_hidden == 0:
            shared = None
        if out is None:
            out = torch.empty((T, p.dim), dtype=_TORCH_OF[p.out_dtype], device=x.device)
        _check_tensor("out", out, _TORCH_OF[p.out_dtype], (T, p.dim), x.device)
        if expert_counts is not None:
            _check_tensor("expert_counts", expert_counts, torch.int32, (p.n_routed,), x.device)
        ew, sw = _weights(experts), _weights(shared)
        fn, name = ((self.lib.moe_layer_forward_train, "moe_layer_forward_train") if train
                    else (self.lib.moe_layer_forward, "moe_layer_forward"))
        st = fn(self.handle, _ptr(x), T, _ptr(gate_w), _ptr(sel_bias), ctypes.byref(ew),
                None if sw is None else ctypes.byref(sw), _ptr(out), _ptr(expert_counts), _stream_handle(stream))
        self._check(st, name)
        return out

    def backward(self, x, gate_w, sel_bias, experts, shared, d_out, stream=None, saved=False):
        """Gradients of sum(d_out * forward(...)) (moe_layer_backward); the cfg
        needs backward=True. Returns dict(dx [T, D], d_gate_w [E, D],
        d_gate_up [E, 2H, D], d_down [E, D, H], d_shared_gate_up [2Hs, D],
        d_shared_down [D, Hs]) of fp32 tensors (shared ones None without a
        shared expert). saved=True: moe_layer_backward_saved, which reads the
        gate/up products left by the last forward(train=True) on the same
        inputs instead of recomputing them."""
        p = self.params
        self._check_x(x)
        T = x.shape[0]
        dev = x.device
        _check_tensor("d_out", d_out, torch.float32, (T, p.dim), dev)
        self._check_router_inputs(x, gate_w, sel_bias)
        self._check_weights(x, experts, shared)
        if p.shared_hidden == 0:
            shared = None
        f32 = dict(dtype=torch.float32, device=dev)
        g = dict(dx=torch.empty((T, p.dim), **f32), d_gate_w=torch.empty((p.n_routed, p.dim), **f32),
                 d_gate_up=torch.empty((p.n_routed, 2 * p.hidden, p.dim), **f32),
                 d_down=torch.empty((p.n_routed, p.dim, p.hidden), **f32),
                 d_shared_gate_up=None, d_shared_down=None)
        dg = MoeWeightGrads(g["d_gate_up"].data_ptr(), g["d_down"].data_ptr())
        dsg = None
        if p.shared_hidden > 0:
            g["d_shared_gate_up"] = torch.empty((2 * p.shared_hidden, p.dim), **f32)
            g["d_shared_down"] = torch.empty((p.dim, p.shared_hidden), **f32)
            dsg = MoeWeightGrads(g["d_shared_gate_up"].data_ptr(), g["d_shared_down"].data_ptr())
        ew, sw = _weights(experts), _weights(shared)
        fn, name = ((self.lib.moe_layer_backward_saved, "moe_layer_backward_saved") if saved
                    else (self.lib.moe_layer_backward, "moe_layer_backward"))
        st = fn(self.handle, _ptr(x), T, _ptr(gate_w), _ptr(sel_bias), ctypes.byref(ew),
                None if sw is None else ctypes.byref(sw), _ptr(d_out), _ptr(g["dx"]), _ptr(g["d_gate_w"]),
                ctypes.byref(dg), None if dsg is None else ctypes.byref(dsg), _stream_handle(stream))
        self._check(st, name)
        return g

    def router(self, x, gate_w, sel_bias, stream=None):
        """(topk_idx [T, K] int32, topk_gate [T, K] fp32, expert_counts [E] int32)."""
        p = self.params
        self._check_x(x)
        self._check_router_inputs(x, gate_w, sel_bias)
        T = x.shape[0]
        idx = torch.empty((T, p.top_k), dtype=torch.int32, device=x.device)
        gate = torch.empty((T, p.top_k), dtype=torch.float32, device=x.device)
        counts = torch.empty((p.n_routed,), dtype=torch.int32, device=x.device)
        st = self.lib.moe_router_forward(self.handle, _ptr(x), T, _ptr(gate_w), _ptr(sel_bias), _ptr(idx),
                                         _ptr(gate), _ptr(counts), _stream_handle(stream))
        self._check(st, "moe_router_forward")
        return idx, gate, counts

    def dispatch(self, topk_idx, stream=None):
        """(offsets [E+1], row_token [T*K], slot_row [T*K]), all int32."""
        p = self.params
        if not torch.is_tensor(topk_idx) or topk_idx.dim() != 2:
            raise ValueError(f"topk_idx must be an int32 cuda tensor [T, {p.top_k}]")
        T = topk_idx.shape[0]
        dev = topk_idx.device
        _check_tensor("topk_idx", topk_idx, torch.int32, (T, p.top_k), dev)
        offsets = torch.empty((p.n_routed + 1,), dtype=torch.int32, device=dev)
        row_token = torch.empty((max(T * p.top_k, 1),), dtype=torch.int32, device=dev)
        slot_row = torch.empty((max(T * p.top_k, 1),), dtype=torch.int32, device=dev)
        st = self.lib.moe_dispatch_forward(self.handle, _ptr(topk_idx), T, _ptr(offsets),
                                           _ptr(row_token), _ptr(slot_row), _stream_handle(stream))
        self._check(st, "moe_dispatch_forward")
        return offsets, row_token[:T * p.top_k], slot_row[:T * p.top_k]


def _check_counts(expert_counts):
    if not torch.is_tensor(expert_counts) or expert_counts.dim() != 1 or not expert_counts.is_cuda:
        raise ValueError("expert_counts must be a 1-d int32 cuda tensor [E]")
    _check_tensor("expert_counts", expert_counts, torch.int32, (expert_counts.shape[0],), expert_counts.device)
    return expert_counts.shape[0]


def bias_update(expert_counts, sel_bias, gamma: float, stream=None):
    """moe_bias_update: sel_bias [E] fp32 (device, updated in place) from
    expert_counts [E] int32 (device)."""
    E = _check_counts(expert_counts)
    _check_tensor("sel_bias", sel_bias, torch.float32, (E,), expert_counts.device)
    st = load_library().moe_bias_update(_ptr(expert_counts), E, float(gamma),
                                        _ptr(sel_bias), _stream_handle(stream))
    if st != MOE_OK:
        raise MoEError(st, "moe_bias_update")
    return sel_bias


def load_stats(expert_counts, stream=None):
    """moe_load_stats: tensor [3] fp32 = (std of load, mean (load - 1/E)^2,
    max violation) from expert_counts [E] int32 (device)."""
    E = _check_counts(expert_counts)
    stats = torch.empty((3,), dtype=torch.float32, device=expert_counts.device)
    st = load_library().moe_load_stats(_ptr(expert_counts), E, _ptr(stats), _stream_handle(stream))
    if st != MOE_OK:
        raise MoEError(st, "moe_load_stats")
    return stats


def debug_status():
    """moe_debug_status: (site, value) of the first bounds violation since the
    last call (0, 0 when none); the library must be the debug build."""
    site, value = ctypes.c_int(), ctypes.c_int()
    st = load_library().moe_debug_status(ctypes.byref(site), ctypes.byref(value))
    if st != MOE_OK:
        raise MoEError(st, "moe_debug_status")
    return site.value, value.value


def layer_forward_noalloc(params: MoeParams, x, gate_w, sel_bias, experts, shared, out=None,
                          expert_counts=None, stream=None):
    """moe_layer_forward_noalloc: the layer forward on the library's fixed
    per-GPU scratch array (no cfg, no device allocation by the library).
    The tensors are checked against params as for MoELayer.forward; out is
    allocated here by torch when not given."""
    chk = MoELayer.__new__(MoELayer)  # the checks only, without a cfg
    chk.params = params
    chk._check_x(x)
    T = x.shape[0]
    chk._check_router_inputs(x, gate_w, sel_bias)
    chk._check_weights(x, experts, shared)
    if params.shared_hidden == 0:
        shared = None
    if out is None:
        out = torch.empty((T, params.dim), dtype=_TORCH_OF[params.out_dtype], device=x.device)
    _check_tensor("out", out, _TORCH_OF[params.out_dtype], (T, params.dim), x.device)
    if expert_counts is not None:
        _check_tensor("expert_counts", expert_counts, torch.int32, (params.n_routed,), x.device)
    ew, sw = _weights(experts), _weights(shared)
    st = load_library().moe_layer_forward_noalloc(ctypes.byref(params), _ptr(x), T, _ptr(gate_w), _ptr(sel_bias),
                                                  ctypes.byref(ew), None if sw is None else ctypes.byref(sw),
                                                  _ptr(out), _ptr(expert_counts), _stream_handle(stream))
    if st != MOE_OK:
        raise MoEError(st, "moe_layer_forward_noalloc")
    return out


BALANCE_STATS = ("load_std", "load_loss", "max_violation", "importance_std", "importance_loss",
                 "device_load_std", "device_load_loss", "device_importance_std", "device_importance_loss")


def balance_stats(expert_counts, score_sum, n_devices: int = 1, stream=None):
    """moe_balance_stats: tensor [9] fp32 (names in BALANCE_STATS) from
    expert_counts [E] int32 and score_sum [E] fp32 (device)."""
    E = _check_counts(expert_counts)
    _check_tensor("score_sum", score_sum, torch.float32, (E,), expert_counts.device)
    stats = torch.empty((len(BALANCE_STATS),), dtype=torch.float32, device=expert_counts.device)
    st = load_library().moe_balance_stats(_ptr(expert_counts), _ptr(score_sum), E, int(n_devices), _ptr(stats),
                                          _stream_handle(stream))
    if st != MOE_OK:
        raise MoEError(st, "moe_balance_stats")
    return stats


def quantize_e4m3_1x128(x, stream=None):
    """moe_quantize_e4m3_1x128: (codes uint8 [rows, cols], scales fp32
    [rows, cols/128]) of a contiguous cuda bf16 tensor x [rows, cols]."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous cuda bf16 tensor [rows, cols]")
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, max(cols // 128, 1)), dtype=torch.float32, device=x.device)
    st = load_library().moe_quantize_e4m3_1x128(_ptr(x), rows, cols, _ptr(codes), _ptr(scales),
                                                _stream_handle(stream))
    if st != MOE_OK:
        raise MoEError(st, "moe_quantize_e4m3_1x128")
    return codes, scales[:, :cols // 128]
