"""Shared helpers of the parity tests: run a workload through the C ABI on
the GPU and through the oracle on the CPU, from the same seeded inputs, and
compare what the tolerances of the method fix:

  * Muon update delta per matrix and step: relative Frobenius error
    <= 2e-2 with bf16 Newton-Schulz, <= 1e-4 with fp32;
  * AdamW p, m, v per element: |x - x_ref| <= 1e-5 |x_ref| + 1e-9, and m, v
    also relative-only (exact zeros skipped) at 1e-5;
  * global gradient norm: 1e-5 relative;
  * Muon momentum buffers: fp32 rounding of the same recurrence.
"""

from __future__ import annotations

import math
import sys
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

import oracle as O
import workloads as W

BF16_TOL = 2e-2
FP32_TOL = 1e-4


def say(*a):
    print("[parity]", *a, flush=True)
    sys.stdout.flush()


def oracle_hparams(w: W.Workload, ns_steps: Optional[int] = None, **kw) -> O.HParams:
    hp = O.HParams()
    hp.param_storage = w.param_storage
    for k, v in W.hparams_for(w).items():
        setattr(hp, k, v)
    for k, v in kw.items():
        setattr(hp, k, v)
    if ns_steps is not None:
        hp.muon_ns_steps = ns_steps
    return hp


def lib_hparams(M, hp: O.HParams, ns_precision: str):
    return M.muon_adamw_default_hparams(
        lr=hp.lr, muon_lr_scale=hp.muon_lr_scale, muon_momentum=hp.muon_momentum,
        muon_nesterov=1 if hp.muon_nesterov else 0, muon_ns_steps=hp.muon_ns_steps,
        ns_coeffs=hp.ns_coeffs, ns_precision=ns_precision, ns_eps=hp.ns_eps,
        beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps, weight_decay=hp.weight_decay,
        muon_weight_decay=hp.muon_weight_decay, max_grad_norm=hp.max_grad_norm,
        lr_schedule=hp.lr_schedule, warmup_steps=hp.warmup_steps, total_steps=hp.total_steps,
        min_lr_rate=hp.min_lr_rate)


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    if den == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / den)


def check_adamw(p, m, v, rp, rm, rv, where: str, m_terms=None):
    """The stated gate on p, m, v (1e-5 relative + 1e-9 absolute), plus two
    stricter ones that the floor would make vacuous for tiny moments: v
    relative-only (a sum of non-negative terms, so no cancellation), and m
    relative to the same moving average taken over |g'| (m itself may cancel
    to near zero, and its rounding error is bounded by the magnitudes of the
    terms summed so far, not by |m|)."""
    p = np.asarray(p, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    rp = np.asarray(rp, np.float64)
    rm = np.asarray(rm, np.float64)
    rv = np.asarray(rv, np.float64)
    for name, x, r in (("p", p, rp), ("m", m, rm), ("v", v, rv)):
        bad = np.abs(x - r) > 1e-5 * np.abs(r) + 1e-9
        assert not bad.any(), "%s AdamW %s: %d elements off, worst %r vs %r" % (
            where, name, int(bad.sum()), x[bad][:3], r[bad][:3])
    nz = rv != 0.0
    rel = np.abs(v[nz] - rv[nz]) / np.abs(rv[nz])
    assert rel.size == 0 or rel.max() <= 1e-5, "%s AdamW v relative %g" % (where, rel.max())
    scale = np.abs(rm) if m_terms is None else np.asarray(m_terms, np.float64)
    nz = scale != 0.0
    rel = np.abs(m[nz] - rm[nz]) / scale[nz]
    assert rel.size == 0 or rel.max() <= 1e-5, "%s AdamW m relative %g" % (where, rel.max())


def check_adamw_bf16(p, m, v, rp32, rm, rv, rp16, where: str, m_terms=None) -> float:
    """bf16-stored parameters: m and v as check_adamw; p must be the bfloat16
    rounding (ties to even) of some value within the stated gate of the
    oracle's unrounded result -- rounding is monotone, so p lies between the
    roundings of the gate's two ends (only near a rounding midpoint are both
    neighbours allowed).  rp32: the oracle's result with float32 storage
    (rounding error 6e-8, far inside the gate); rp16: the oracle's own bf16
    result.  Returns the fraction of elements equal to rp16."""
    check_adamw(rp32, m, v, rp32, rm, rv, where, m_terms)
    p = np.asarray(p, np.float32)
    r = np.asarray(rp32, np.float64)
    d = 1e-5 * np.abs(r) + 1e-9
    lo = O.bf16_round_f64(r - d)
    hi = O.bf16_round_f64(r + d)
    bad = (p < lo) | (p > hi)
    assert not bad.any(), "%s AdamW bf16 p: %d elements outside the rounding window, e.g. %r " \
        "not in [%r, %r]" % (where, int(bad.sum()), p[bad][:3], lo[bad][:3], hi[bad][:3])
    assert np.all(O.bf16_round(p) == p), "%s: p holds values that are not bfloat16" % where
    return float(np.mean(p == np.asarray(rp16, np.float32)))


@dataclass
class GpuRun:
    """Device tensors of one workload and the library objects around them."""
    w: W.Workload
    plan: object
    groups: List[int]
    params: List
    grads: List
    state: object
    hp: object
    workspace: object
    deltas: List
    norm_out: object


def setup_gpu(M, torch, w: W.Workload, hp: O.HParams, ns_precision: str, backend: str = "numpy",
              deltas: str = "all", overlap: bool = False):
    """Allocate and seed a workload on cuda:0.  deltas: 'all', 'none' or a set
    of entry indices that get a delta output buffer; overlap: the plan's
    overlap_groups (the workspace is sized for that plan)."""
    dev = torch.device("cuda", 0)
    table = list(zip(w.names, w.shapes, w.trainable))
    plan = M.muon_adamw_plan(table, mode=W.mode_id(w), param_dtype=w.param_storage,
                             overlap_groups=overlap)
    pdt = torch.bfloat16 if w.param_storage == "bf16" else torch.float32
    n = len(w.params)
    groups = [M.muon_adamw_plan_entry(plan, i)["group"] for i in range(n)]
    params, grads, dl = [None] * n, [None] * n, [None] * n
    state = M.State(n)
    for i, spec in enumerate(w.params):
        if groups[i] == M.MA_GROUP_NONE:
            continue
        if backend == "numpy":
            params[i] = torch.from_numpy(W.np_param(w, i)).to(dev).to(pdt)
        else:
            params[i] = W.torch_param(w, i, dev).to(pdt)
        grads[i] = torch.empty(spec.shape, dtype=pdt, device=dev)
        if groups[i] == M.MA_GROUP_MUON:
            if backend == "numpy":
                state.muon_momentum[i] = torch.from_numpy(W.np_momentum(w, i)).to(dev)
            else:
                state.muon_momentum[i] = W.torch_momentum(w, i, dev)
            if deltas == "all" or (deltas != "none" and i in deltas):
                dl[i] = torch.empty(spec.shape, dtype=torch.float32, device=dev)
        else:
            state.adam_m[i] = torch.zeros(spec.shape, dtype=torch.float32, device=dev)
            state.adam_v[i] = torch.zeros(spec.shape, dtype=torch.float32, device=dev)
    lhp = lib_hparams(M, hp, ns_precision)
    ws = torch.empty(M.muon_adamw_workspace_size(plan, lhp.ns_precision), dtype=torch.uint8, device=dev)
    norm_out = torch.empty(1, dtype=torch.float32, device=dev)
    return GpuRun(w, plan, groups, params, grads, state, lhp, ws, dl, norm_out)


def fill_grads(run: GpuRun, torch, step: int, backend: str = "numpy"):
    dev = torch.device("cuda", 0)
    for i, g in enumerate(run.grads):
        if g is None:
            continue
        if backend == "numpy":
            g.copy_(torch.from_numpy(W.np_grad(run.w, step, i)).to(dev))
        else:
            W.torch_grad(run.w, step, i, dev, out=g)


def gpu_step(M, torch, run: GpuRun):
    M.muon_adamw_step(run.plan, run.params, run.grads, run.state, run.hp, run.workspace,
                      grad_norm_out=run.norm_out, muon_update_out=run.deltas)
    torch.cuda.synchronize()


def host(t) -> np.ndarray:
    """A device tensor's values on the host (bfloat16 widened to float32)."""
    t = t.detach()
    if str(t.dtype) == "torch.bfloat16":
        t = t.float()
    return t.cpu().numpy()


def oracle_norm_of_device_grads(run: GpuRun) -> float:
    """The oracle's global norm over every trainable gradient, each read back
    from the device as it is consumed."""
    return O.global_grad_norm(host(g) for g in run.grads if g is not None)


def ragged_workload():
    """Ragged Muon shapes in both orientations around tile edges, odd AdamW
    sizes, a frozen entry and a 2-D norm weight (AdamW by name)."""
    shapes = [(1, 7), (7, 1), (33, 65), (65, 33), (130, 300), (300, 130), (256, 256),
              (257, 513), (513, 257), (64, 256), (3, 1000), (129, 129)]
    params = [W.ParamSpec("action_expert.layers.%d.r.weight" % i, s) for i, s in enumerate(shapes)]
    params += [W.ParamSpec("vlm.bias", (3,)), W.ParamSpec("vlm.w", (5, 7)),
               W.ParamSpec("vlm.big", (16385,)), W.ParamSpec("vlm.cube", (4, 4, 4)),
               W.ParamSpec("vlm.frozen", (9, 9), trainable=False),
               W.ParamSpec("action_expert.layers.0.norm.weight", (40, 40))]
    return W.Workload("ragged_small", seed=7, steps=2, ns_precision="bf16", params=params,
                      grad_std=1e-3)


def known_svd_muon_delta_rows(ks, rows, hp: O.HParams, m: int, n: int, norm: float):
    """Expected Muon update of the first step from a fresh state for the
    gradient G = U diag(sigma) V^T of `ks` (canonical r x c; stored m x n),
    at canonical rows `rows`, from the oracle's steps applied to the known
    spectrum: the clip factor, the momentum direction (a multiple of G with
    a zero buffer), the Frobenius normalisation, the NS map of every singular
    value, and the rate.  Returns a (len(rows), c) float64 array."""
    coef = O.clip_coefficient(norm, hp.max_grad_norm)
    u, _ = O.nesterov_momentum(np.ones(1), np.zeros(1), coef, hp.muon_momentum, hp.muon_nesterov)
    fac = float(u[0])                      # u = fac * G
    fro = fac * math.sqrt(float(np.dot(ks.sigma, ks.sigma)))
    x0 = fac * ks.sigma / (fro + hp.ns_eps)
    phi = O.ns_spectral_map(x0, hp.muon_ns_steps, hp.ns_coeffs)
    rate = (O.scheduled_lr(hp, 1) * float(hp.muon_lr_scale) *
            float(O.lr_shape_scale(m, n)))
    return np.stack([W.np_known_svd_row(ks, i, rate * phi) for i in rows])
