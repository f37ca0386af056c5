"""Python binding of the MI355X hybrid MuonAdamW optimizer step.

Same names as the C ABI in include/muon_adamw.h; argument marshalling only.
Device memory and streams come from PyTorch (tensors' data pointers and
`torch.cuda.current_stream()`); every step of the optimizer runs in the HIP
library libmuon_adamw.so, which must have been built (there is no fallback).

`MuonAdamW` is a small convenience holder: it allocates the optimizer state
and workspace as torch tensors and calls `muon_adamw_step`.
"""

from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional, Sequence, Tuple

from . import _abi
from ._abi import (MA_ERR_CAPTURE, MA_ERR_HIP, MA_ERR_INVALID_ARG, MA_ERR_SHAPE, MA_ERR_UNSUPPORTED,  # noqa: F401
                   MA_ERR_WORKSPACE, MA_GROUP_ADAMW, MA_GROUP_MUON, MA_GROUP_NONE,
                   MA_LR_CONSTANT, MA_LR_COSINE_MIN, MA_MODE_ADAMW, MA_MODE_MUON_ADAMW,
                   MA_NOALLOC_SCRATCH_BYTES, MA_NS_BF16, MA_NS_FP32, MA_OK, MA_PARAM_BF16,
                   MA_PARAM_FP32)

__all__ = [
    "MuonAdamWError", "Plan", "State",
    "muon_adamw_default_hparams", "muon_adamw_plan", "muon_adamw_plan_size",
    "muon_adamw_plan_entry", "muon_adamw_plan_dump", "muon_adamw_workspace_size",
    "muon_adamw_step", "muon_adamw_step_profiled", "muon_adamw_step_noalloc",
    "muon_adamw_plan_free", "muon_adamw_last_error",
    "muon_adamw_version", "MuonAdamW", "load_library",
]


class MuonAdamWError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("%s (code %d)" % (message, code))
        self.code = code


def load_library():
    return _abi.load()


def _check(rc: int, what: str):
    if rc != MA_OK:
        msg = _abi.load().muon_adamw_last_error().decode("utf-8", "replace")
        raise MuonAdamWError(rc, "%s: %s" % (what, msg))


def muon_adamw_last_error() -> str:
    return _abi.load().muon_adamw_last_error().decode("utf-8", "replace")


def muon_adamw_version() -> str:
    return _abi.load().muon_adamw_version().decode()


def muon_adamw_default_hparams(**overrides) -> _abi.ma_hparams:
    """The library's defaults, with keyword overrides (field names of
    ma_hparams; `ns_coeffs` takes a 3-sequence, `ns_precision` also accepts
    'bf16' / 'fp32', `lr_schedule` 'constant' / 'cosine_with_min_lr')."""
    hp = _abi.ma_hparams()
    _check(_abi.load().muon_adamw_default_hparams(C.byref(hp)), "muon_adamw_default_hparams")
    for k, v in overrides.items():
        if k == "ns_coeffs":
            for i in range(3):
                hp.ns_coeffs[i] = float(v[i])
        elif k == "ns_precision" and isinstance(v, str):
            hp.ns_precision = {"bf16": MA_NS_BF16, "fp32": MA_NS_FP32}[v]
        elif k == "lr_schedule" and isinstance(v, str):
            hp.lr_schedule = {"constant": MA_LR_CONSTANT, "cosine_with_min_lr": MA_LR_COSINE_MIN}[v]
        elif k in ("muon_nesterov", "muon_ns_steps", "ns_precision", "lr_schedule",
                   "warmup_steps", "total_steps"):
            setattr(hp, k, int(v))
        else:
            if not hasattr(hp, k):
                raise KeyError("unknown hyperparameter %r" % k)
            setattr(hp, k, float(v))
    return hp


class Plan:
    """Owning handle of an ma_plan (freed with the object)."""

    def __init__(self, handle: int, names: Sequence[str], shapes: Sequence[Tuple[int, ...]],
                 param_dtype: int = MA_PARAM_FP32):
        self.handle = C.c_void_p(handle)
        self.names = list(names)
        self.shapes = [tuple(s) for s in shapes]
        self.param_dtype = param_dtype

    def __del__(self):
        try:
            if self.handle and self.handle.value:
                _abi.load().muon_adamw_plan_free(self.handle)
                self.handle = C.c_void_p(0)
        except Exception:
            pass


def muon_adamw_plan(table: Sequence[Tuple[str, Sequence[int], bool]],
                    mode: int = MA_MODE_MUON_ADAMW,
                    moonlight_coefficient: float = 0.2, overlap_groups: bool = False,
                    param_dtype="fp32") -> Plan:
    """Route a parameter table [(name, shape, trainable), ...] (host only).
    overlap_groups: run the AdamW group concurrently with the Muon group.
    param_dtype: storage of parameters and gradients, 'fp32' or 'bf16' (or
    MA_PARAM_*); optimizer states are float32 either way."""
    if isinstance(param_dtype, str):
        param_dtype = {"fp32": MA_PARAM_FP32, "bf16": MA_PARAM_BF16}[param_dtype]
    n = len(table)
    descs = (_abi.ma_param_desc * max(n, 1))()
    keep = []
    for i, (name, shape, trainable) in enumerate(table):
        nb = name.encode("utf-8")
        sh = (C.c_int64 * max(len(shape), 1))(*[int(s) for s in shape])
        keep.append((nb, sh))
        descs[i].name = nb
        descs[i].ndim = len(shape)
        descs[i].shape = C.cast(sh, C.POINTER(C.c_int64))
        descs[i].trainable = 1 if trainable else 0
    opts = _abi.ma_plan_opts(int(mode), float(moonlight_coefficient), 1 if overlap_groups else 0,
                             int(param_dtype))
    out = C.c_void_p()
    _check(_abi.load().muon_adamw_plan(descs, n, C.byref(opts), C.byref(out)), "muon_adamw_plan")
    return Plan(out.value, [t[0] for t in table], [tuple(t[1]) for t in table], int(param_dtype))


def muon_adamw_plan_free(plan: Plan):
    plan.__del__()


def muon_adamw_plan_size(plan: Plan) -> int:
    n = C.c_int32()
    _check(_abi.load().muon_adamw_plan_size(plan.handle, C.byref(n)), "muon_adamw_plan_size")
    return n.value


def muon_adamw_plan_entry(plan: Plan, i: int) -> Dict[str, object]:
    e = _abi.ma_plan_entry()
    _check(_abi.load().muon_adamw_plan_entry(plan.handle, int(i), C.byref(e)),
           "muon_adamw_plan_entry")
    return {f: getattr(e, f) for f, _ in e._fields_}


def muon_adamw_plan_dump(plan: Plan) -> str:
    lib = _abi.load()
    n = C.c_size_t()
    _check(lib.muon_adamw_plan_dump(plan.handle, None, 0, C.byref(n)), "muon_adamw_plan_dump")
    buf = C.create_string_buffer(n.value + 1)
    _check(lib.muon_adamw_plan_dump(plan.handle, buf, n.value + 1, C.byref(n)),
           "muon_adamw_plan_dump")
    return buf.raw[:n.value].decode("utf-8")


def muon_adamw_workspace_size(plan: Plan, ns_precision: int = MA_NS_BF16) -> int:
    n = C.c_size_t()
    _check(_abi.load().muon_adamw_workspace_size(plan.handle, int(ns_precision), C.byref(n)),
           "muon_adamw_workspace_size")
    return n.value


def _ptr(x, bf16: bool = False, numel: Optional[int] = None, what: str = "tensor") -> Optional[int]:
    """Device address of a contiguous torch tensor (or an int, taken as is):
    float32, or bfloat16 where `bf16` (parameters and gradients of a bf16
    plan).  With `numel` given, a tensor must hold exactly that many
    elements (a uint8 tensor standing for raw memory: at least that many
    elements' bytes), so a mis-sized or mis-ordered list is refused before
    the library could read or write past a buffer."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError("expected a torch tensor, an int address or None")
    want = torch.bfloat16 if bf16 else torch.float32
    if x.dtype != want and x.dtype != torch.uint8:
        raise TypeError("%s must be %s (got %s)" % (what, want, x.dtype))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    if numel is not None:
        if x.dtype == torch.uint8:
            need = numel * (2 if bf16 else 4)
            if x.numel() < need:
                raise ValueError("%s: %d bytes, the plan needs %d" % (what, x.numel(), need))
        elif x.numel() != numel:
            raise ValueError("%s: %d elements, the plan says %d" % (what, x.numel(), numel))
    if x.device.type != "cuda":
        raise ValueError("%s must live on the GPU" % what)
    return x.data_ptr()


def _numel(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def _ptr_array(xs, n: int, bf16: bool = False, plan: Optional["Plan"] = None,
               what: str = "tensor"):
    """ctypes array of n addresses; with `plan`, each tensor is checked
    against its entry's element count."""
    arr = (C.c_void_p * max(n, 1))()
    if xs is not None:
        if plan is not None and len(xs) > n:
            raise ValueError("%s list has %d items for %d plan entries" % (what, len(xs), n))
        for i, x in enumerate(xs):
            numel = _numel(plan.shapes[i]) if plan is not None else None
            arr[i] = _ptr(x, bf16, numel, "%s %d" % (what, i))
    return arr


class State:
    """Caller-owned optimizer state: per-entry momentum (Muon) and moments
    (AdamW) tensors, plus the step counter: the host int `step`, or, when
    `device_step` is set (a one-element int64 CUDA tensor or an address),
    that device counter, which each step reads and advances on the GPU."""

    def __init__(self, n: int):
        self.muon_momentum: List = [None] * n
        self.adam_m: List = [None] * n
        self.adam_v: List = [None] * n
        self.step = 0
        self.device_step = None


def _step_ptr(x) -> int:
    if x is None or isinstance(x, int):
        return int(x or 0)
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype != torch.int64 or x.numel() != 1:
        raise TypeError("device_step must be a one-element int64 tensor or an address")
    if x.device.type != "cuda":
        raise ValueError("device_step must live on the GPU")
    return x.data_ptr()


def muon_adamw_step(plan: Plan, params, grads, state: State, hp: _abi.ma_hparams,
                    workspace, stream=None, grad_norm_out=None, muon_update_out=None) -> None:
    """One optimizer step on `stream` (a torch.cuda.Stream, a raw hipStream_t
    int, or None for torch's current stream).  Asynchronous."""
    _step(plan, params, grads, state, hp, workspace, stream, grad_norm_out, muon_update_out, None)


def muon_adamw_step_profiled(plan: Plan, params, grads, state: State, hp: _abi.ma_hparams,
                             workspace, phase_events, stream=None, grad_norm_out=None,
                             muon_update_out=None) -> None:
    """muon_adamw_step that also records MA_PROFILE_EVENTS caller-created
    hipEvent_t handles (ints) at its phase boundaries."""
    _step(plan, params, grads, state, hp, workspace, stream, grad_norm_out, muon_update_out,
          phase_events)


def muon_adamw_step_noalloc(plan: Plan, params, grads, state: State, hp: _abi.ma_hparams,
                            stream=None, grad_norm_out=None, muon_update_out=None) -> None:
    """muon_adamw_step without a workspace and without any allocation: the
    library's per-device scratch (MA_NOALLOC_SCRATCH_BYTES) serves, every
    kernel runs on `stream`, and calls on one GPU must not overlap."""
    _step(plan, params, grads, state, hp, None, stream, grad_norm_out, muon_update_out, None)


def _step(plan, params, grads, state, hp, workspace, stream, grad_norm_out, muon_update_out,
          phase_events):
    n = len(plan.names)
    st = _abi.ma_state()
    mm = _ptr_array(state.muon_momentum, n, plan=plan, what="muon_momentum")
    am = _ptr_array(state.adam_m, n, plan=plan, what="adam_m")
    av = _ptr_array(state.adam_v, n, plan=plan, what="adam_v")
    st.muon_momentum = C.cast(mm, C.POINTER(C.c_void_p))
    st.adam_m = C.cast(am, C.POINTER(C.c_void_p))
    st.adam_v = C.cast(av, C.POINTER(C.c_void_p))
    st.step = int(state.step)
    st.device_step = _step_ptr(getattr(state, "device_step", None)) or None
    bf16 = getattr(plan, "param_dtype", MA_PARAM_FP32) == MA_PARAM_BF16
    pa = _ptr_array(params, n, bf16, plan=plan, what="param")
    ga = _ptr_array(grads, n, bf16, plan=plan, what="grad")
    ua = (_ptr_array(muon_update_out, n, plan=plan, what="muon_update_out")
          if muon_update_out is not None else None)
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    if workspace is None:
        ws_ptr, ws_bytes = 0, 0          # the allocation-free step: no workspace
    elif isinstance(workspace, tuple):
        ws_ptr, ws_bytes = int(workspace[0]), int(workspace[1])
    else:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        # (an unknown precision is left for the library to report)
        need = (muon_adamw_workspace_size(plan, hp.ns_precision)
                if hp.ns_precision in (MA_NS_BF16, MA_NS_FP32) else 0)
        if ws_bytes < need:
            raise ValueError("workspace of %d bytes, the plan needs %d" % (ws_bytes, need))
        if workspace.device.type != "cuda":
            raise ValueError("workspace must live on the GPU")
    ua = C.cast(ua, C.POINTER(C.c_void_p)) if ua is not None else None
    args = (plan.handle, pa, ga, C.byref(st), C.byref(hp), C.c_void_p(ws_ptr), ws_bytes,
            C.c_void_p(stream), C.c_void_p(_ptr(grad_norm_out, numel=1, what="grad_norm_out") or 0),
            ua)
    if workspace is None:
        rc = _abi.load().muon_adamw_step_noalloc(args[0], args[1], args[2], args[3], args[4],
                                                 args[7], args[8], args[9])
    elif phase_events is None:
        rc = _abi.load().muon_adamw_step(*args)
    else:
        ev = (C.c_void_p * _abi.MA_PROFILE_EVENTS)(*[int(e) for e in phase_events])
        rc = _abi.load().muon_adamw_step_profiled(*args, C.cast(ev, C.POINTER(C.c_void_p)))
    _check(rc, "muon_adamw_step")
    state.step = st.step


class MuonAdamW:
    """Plan + state + workspace for a list of (name, tensor, trainable).

    Tensors are float32 (or, all of them, bfloat16: the bf16 parameter
    storage) CUDA tensors owned by the caller; gradients are passed to
    `step`.  State tensors are float32 and start at zero."""

    def __init__(self, named_params: Sequence[Tuple[str, object, bool]],
                 mode: int = MA_MODE_MUON_ADAMW, overlap_groups: bool = False, **hparams):
        import torch
        self.names = [n for n, _, _ in named_params]
        self.params = [p for _, p, _ in named_params]
        bf16 = any(p is not None and p.dtype == torch.bfloat16 for p in self.params)
        self.plan = muon_adamw_plan([(n, tuple(p.shape), t) for n, p, t in named_params], mode,
                                    overlap_groups=overlap_groups,
                                    param_dtype="bf16" if bf16 else "fp32")
        self.hp = muon_adamw_default_hparams(**hparams)
        self.state = State(len(self.names))
        self.groups = []
        for i, p in enumerate(self.params):
            g = muon_adamw_plan_entry(self.plan, i)["group"]
            self.groups.append(g)
            if g == MA_GROUP_MUON:
                self.state.muon_momentum[i] = torch.zeros_like(p, dtype=torch.float32)
            elif g == MA_GROUP_ADAMW:
                self.state.adam_m[i] = torch.zeros_like(p, dtype=torch.float32)
                self.state.adam_v[i] = torch.zeros_like(p, dtype=torch.float32)
        dev = next((p.device for p in self.params if p is not None), torch.device("cuda"))
        nbytes = muon_adamw_workspace_size(self.plan, self.hp.ns_precision)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def step(self, grads, stream=None, grad_norm_out=None, muon_update_out=None):
        muon_adamw_step(self.plan, self.params, grads, self.state, self.hp, self.workspace,
                        stream, grad_norm_out, muon_update_out)
