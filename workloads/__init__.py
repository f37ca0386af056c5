"""Synthetic workloads and seeded input generators.

This module holds parameter tables (names, shapes, trainable flags), the
hyperparameters each workload runs with, and seeded random inputs.  It holds
none of the optimizer's arithmetic, so both the oracle side (tests, the CPU
baseline) and the GPU side (tests, the benchmark) may draw from it.

Names follow the layout of the model family on the OpenDM training-stack page
(an action expert with `layers`, a VLM backbone whose token embedding is frozen);
the page gives no concrete tables, so these are synthetic and sized by the
workload definitions below.

Two generator back ends produce the same *kind* of values from the same seeds:
  * numpy: PCG64 streams `default_rng([seed, kind, step, index])`, float32;
  * torch: one Philox generator on the target device per tensor, seeded by a
    hash of the same tuple.  Used where host generation of billions of values
    would dominate the run (the full-size hybrid workload).
The two back ends do not produce equal values; a run uses one of them for
both sides of a comparison (the oracle reads the device tensors' copies).
"""

from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

KIND_PARAM, KIND_GRAD, KIND_MOMENTUM = 0, 1, 2


@dataclass(frozen=True)
class ParamSpec:
    name: str
    shape: Tuple[int, ...]
    trainable: bool = True

    @property
    def numel(self) -> int:
        n = 1
        for d in self.shape:
            n *= d
        return n


@dataclass
class Workload:
    name: str
    seed: int
    steps: int
    ns_precision: str                 # "bf16" or "fp32"
    params: List[ParamSpec]
    grad_std: float
    weight_std: float = 0.02
    grad_row_scale: Optional[Tuple[float, float]] = None   # log-uniform per stored row
    spike: Optional[Tuple[int, float]] = None               # (rank, entry std)
    momentum_init_std: float = 0.0
    hparams: Dict[str, object] = field(default_factory=dict)
    description: str = ""
    mode: str = "muon_adamw"          # or "adamw": every trainable tensor to AdamW
    param_storage: str = "fp32"       # or "bf16": parameters and gradients stored as bfloat16

    @property
    def names(self) -> List[str]:
        return [p.name for p in self.params]

    @property
    def shapes(self) -> List[Tuple[int, ...]]:
        return [p.shape for p in self.params]

    @property
    def trainable(self) -> List[bool]:
        return [p.trainable for p in self.params]


# --------------------------------------------------------------------------
# parameter tables
# --------------------------------------------------------------------------

def _action_expert_layers(n_layers: int, hidden: int, kv: int, mlp: int) -> List[ParamSpec]:
    out = []
    for layer in range(n_layers):
        pre = "action_expert.layers.%d." % layer
        out += [
            ParamSpec(pre + "self_attn.q_proj.weight", (hidden, hidden)),
            ParamSpec(pre + "self_attn.k_proj.weight", (kv, hidden)),
            ParamSpec(pre + "self_attn.v_proj.weight", (kv, hidden)),
            ParamSpec(pre + "self_attn.o_proj.weight", (hidden, hidden)),
            ParamSpec(pre + "mlp.gate_proj.weight", (mlp, hidden)),
            ParamSpec(pre + "mlp.up_proj.weight", (mlp, hidden)),
            ParamSpec(pre + "mlp.down_proj.weight", (hidden, mlp)),
        ]
    return out


def tiny_hybrid_fp32() -> Workload:
    """Two action-expert layers (q,k,v,o 256x256; gate,up 1024x256; down
    256x1024: 14 matrices) plus an AdamW group of a 1000x256 embedding, eight
    RMSNorm vectors and four biases of 256; fp32 Newton-Schulz; 3 steps."""
    params = _action_expert_layers(2, 256, 256, 1024)
    params.append(ParamSpec("action_expert.embed_tokens.weight", (1000, 256)))
    for layer in range(2):
        pre = "action_expert.layers.%d." % layer
        for nm in ("input_layernorm", "post_attention_layernorm",
                   "self_attn.q_norm", "self_attn.k_norm"):
            params.append(ParamSpec(pre + nm + ".weight", (256,)))
    for layer in range(2):
        pre = "action_expert.layers.%d." % layer
        for nm in ("q_proj", "k_proj"):
            params.append(ParamSpec(pre + "self_attn." + nm + ".bias", (256,)))
    return Workload("tiny_hybrid_fp32", seed=0, steps=3, ns_precision="fp32",
                    params=params, grad_std=1e-3,
                    description="14 Muon matrices (256-1024) + 259,072 AdamW "
                                "elements, fp32 NS")


def _action_expert_18() -> List[ParamSpec]:
    return _action_expert_layers(18, 1024, 256, 4096)


def ae18_muon_bf16() -> Workload:
    """Muon group only: 18 action-expert layers x {q,o 1024x1024; k,v
    256x1024; gate,up 4096x1024; down 1024x4096} = 126 matrices; bf16 NS;
    gradients N(0,1e-3) times a log-uniform [0.1,10] scale per stored row;
    10 steps."""
    return Workload("ae18_muon_bf16", seed=1, steps=10, ns_precision="bf16",
                    params=_action_expert_18(), grad_std=1e-3,
                    grad_row_scale=(0.1, 10.0),
                    description="126 Muon matrices, 273,678,336 params, bf16 NS")


def _vlm_backbone(n_layers=28, hidden=2048, mlp=8192, vocab=151000) -> List[ParamSpec]:
    out = [ParamSpec("vlm.model.embed_tokens.weight", (vocab, hidden), trainable=False)]
    for layer in range(n_layers):
        pre = "vlm.model.layers.%d." % layer
        out += [
            ParamSpec(pre + "self_attn.q_proj.weight", (hidden, hidden)),
            ParamSpec(pre + "self_attn.k_proj.weight", (hidden, hidden)),
            ParamSpec(pre + "self_attn.v_proj.weight", (hidden, hidden)),
            ParamSpec(pre + "self_attn.o_proj.weight", (hidden, hidden)),
            ParamSpec(pre + "mlp.gate_proj.weight", (mlp, hidden)),
            ParamSpec(pre + "mlp.up_proj.weight", (mlp, hidden)),
            ParamSpec(pre + "mlp.down_proj.weight", (hidden, mlp)),
            ParamSpec(pre + "input_layernorm.weight", (hidden,)),
            ParamSpec(pre + "post_attention_layernorm.weight", (hidden,)),
        ]
    out.append(ParamSpec("vlm.model.norm.weight", (hidden,)))
    return out


def vla_hybrid_bf16() -> Workload:
    """The full hybrid step: the 126-matrix action-expert Muon group plus an
    AdamW group shaped like a 1.9B VLM backbone (28 layers, hidden 2048, MLP
    8192; 253 tensors, 1,879,164,928 elements) and a frozen 151000x2048 token
    embedding; gradients N(0,1e-2) so the clip to 1.0 triggers; bf16 NS."""
    return Workload("vla_hybrid_bf16", seed=2, steps=5, ns_precision="bf16",
                    params=_vlm_backbone() + _action_expert_18(), grad_std=1e-2,
                    description="126 Muon matrices + 253 AdamW tensors "
                                "(2,152,843,264 trainable params), bf16 NS")


def vla_hybrid_fp32ns() -> Workload:
    """vla_hybrid_bf16's parameters and seeds with the NS products in full
    fp32."""
    w = vla_hybrid_bf16()
    w.name = "vla_hybrid_fp32ns"
    w.ns_precision = "fp32"
    w.description = "vla_hybrid parameter set, fp32 NS"
    return w


def vla_hybrid_adamw() -> Workload:
    """The page's default optimizer (optim = adamw) over vla_hybrid_bf16's
    parameters and seeds: all 2,152,843,264 trainable elements through the
    clip and AdamW, under the defaults table's cosine_with_min_lr schedule
    (min_lr_rate 0.1) over 1000 steps."""
    w = vla_hybrid_bf16()
    w.name = "vla_hybrid_adamw"
    w.mode = "adamw"
    w.hparams = {"lr_schedule": "cosine_with_min_lr", "total_steps": 1000, "min_lr_rate": 0.1}
    w.description = "vla_hybrid parameter set, pure AdamW (2,152,843,264 params), cosine schedule"
    return w


def ragged_stress_bf16(clip: bool = True) -> Workload:
    """Large and ragged Muon matrices in one call: 8192x8192, 4096x14336,
    14336x4096, 128x8192 and 64 matrices of 64x256; gradients N(0,1) plus a
    rank-8 spike whose entries have std 100; momentum buffers preloaded
    N(0,1e-2); bf16 NS; 3 steps.  `clip=False` turns the global clip off."""
    params = [
        ParamSpec("action_expert.layers.0.stress_0.weight", (8192, 8192)),
        ParamSpec("action_expert.layers.0.stress_1.weight", (4096, 14336)),
        ParamSpec("action_expert.layers.0.stress_2.weight", (14336, 4096)),
        ParamSpec("action_expert.layers.0.stress_3.weight", (128, 8192)),
    ]
    for j in range(64):
        params.append(ParamSpec("action_expert.layers.1.stress_%d.weight" % j, (64, 256)))
    hp = {} if clip else {"max_grad_norm": 0.0}
    return Workload("ragged_stress_bf16" + ("" if clip else "_noclip"), seed=4,
                    steps=3, ns_precision="bf16", params=params, grad_std=1.0,
                    spike=(8, 100.0), momentum_init_std=1e-2, hparams=hp,
                    description="68 Muon matrices (8192^2 ... 64x256), spiked "
                                "gradients, preloaded momentum")


def vla_hybrid_bf16_mixed() -> Workload:
    """vla_hybrid_bf16 under the page's default precision policy bf16_mixed:
    parameters and gradients stored in bfloat16 (the seeded values rounded
    to bfloat16), float32 optimizer states."""
    w = vla_hybrid_bf16()
    w.name = "vla_hybrid_bf16_mixed"
    w.param_storage = "bf16"
    w.description = "vla_hybrid parameter set, bf16 parameters and gradients, bf16 NS"
    return w


def ns_cost(shape: Tuple[int, ...]) -> float:
    """Partitioning cost of one Muon matrix: the dense flop count of five
    Newton-Schulz steps on its canonical r x c (20 r^2 c + 10 r^3)."""
    r, c = min(shape), max(shape)
    return 20.0 * r * r * c + 10.0 * float(r) ** 3


def lpt_owners(shapes, world: int) -> List[int]:
    """Owner GPU of each matrix, longest processing time first: by falling
    cost (ties in table order), each to the least-loaded GPU (ties to the
    lower index)."""
    order = sorted(range(len(shapes)), key=lambda i: (-ns_cost(shapes[i]), i))
    load = [0.0] * world
    owner = [0] * len(shapes)
    for i in order:
        k = min(range(world), key=lambda j: (load[j], j))
        owner[i] = k
        load[k] += ns_cost(shapes[i])
    return owner


def vla_hybrid_share(rank: int = 0, world: int = 8) -> Workload:
    """One GPU's share of vla_hybrid_bf16 when the step is sharded over
    `world` GPUs by owner-compute: the action-expert matrices that LPT
    assigns to `rank` (whole, as Newton-Schulz needs them), and the rank's
    contiguous 1/world range of the concatenated AdamW elements, as 1-D
    pieces.  Same seed and gradient scale; the clip norm is the share's own
    (the all-reduce of the partial sums is not part of one GPU's work)."""
    muon = _action_expert_18()
    owner = lpt_owners([p.shape for p in muon], world)
    mine = [p for p, o in zip(muon, owner) if o == rank]
    adam = [p for p in _vlm_backbone() if p.trainable]
    total = sum(p.numel for p in adam)
    lo, hi = rank * total // world, (rank + 1) * total // world
    pieces, off = [], 0
    for p in adam:
        a, b = max(lo, off), min(hi, off + p.numel)
        if a < b:
            pieces.append(ParamSpec("%s[%d:%d]" % (p.name, a - off, b - off), (b - a,)))
        off += p.numel
    name = "vla_hybrid_rank%d_of%d" % (rank, world)
    return Workload(name, seed=2, steps=5, ns_precision="bf16", params=pieces + mine,
                    grad_std=1e-2,
                    description="GPU %d of %d: %d Muon matrices (LPT by NS flops) + AdamW "
                                "elements [%d, %d) of %d" % (rank, world, len(mine), lo, hi, total))


WORKLOADS = {
    "tiny_hybrid_fp32": tiny_hybrid_fp32,
    "ae18_muon_bf16": ae18_muon_bf16,
    "vla_hybrid_bf16": vla_hybrid_bf16,
    "vla_hybrid_fp32ns": vla_hybrid_fp32ns,
    "vla_hybrid_adamw": vla_hybrid_adamw,
    "vla_hybrid_bf16_mixed": vla_hybrid_bf16_mixed,
    "vla_hybrid_rank0_of8": lambda: vla_hybrid_share(0, 8),
    "ragged_stress_bf16": ragged_stress_bf16,
    "ragged_stress_bf16_noclip": lambda: ragged_stress_bf16(clip=False),
}


# --------------------------------------------------------------------------
# numpy back end
# --------------------------------------------------------------------------

def _rng(seed: int, kind: int, step: int, index: int) -> np.random.Generator:
    return np.random.default_rng([seed, kind, step, index])


def np_param(w: Workload, index: int) -> np.ndarray:
    spec = w.params[index]
    r = _rng(w.seed, KIND_PARAM, 0, index)
    return (r.standard_normal(spec.shape, dtype=np.float32) * np.float32(w.weight_std))


def np_momentum(w: Workload, index: int) -> np.ndarray:
    spec = w.params[index]
    if w.momentum_init_std == 0.0:
        return np.zeros(spec.shape, np.float32)
    r = _rng(w.seed, KIND_MOMENTUM, 0, index)
    return r.standard_normal(spec.shape, dtype=np.float32) * np.float32(w.momentum_init_std)


def np_grad(w: Workload, step: int, index: int) -> np.ndarray:
    spec = w.params[index]
    r = _rng(w.seed, KIND_GRAD, step, index)
    g = r.standard_normal(spec.shape, dtype=np.float32) * np.float32(w.grad_std)
    if w.grad_row_scale is not None and len(spec.shape) >= 1:
        lo, hi = w.grad_row_scale
        s = np.exp(r.uniform(math.log(lo), math.log(hi), spec.shape[0])).astype(np.float32)
        g *= s.reshape((-1,) + (1,) * (len(spec.shape) - 1))
    if w.spike is not None and len(spec.shape) == 2:
        rank, mag = w.spike
        m, n = spec.shape
        u = r.standard_normal((m, rank), dtype=np.float32)
        v = r.standard_normal((n, rank), dtype=np.float32)
        g += (np.float32(mag / math.sqrt(rank)) * (u @ v.T)).astype(np.float32)
    return g


# --------------------------------------------------------------------------
# torch back end (device-side generation for the large workloads)
# --------------------------------------------------------------------------

def torch_seed(seed: int, kind: int, step: int, index: int) -> int:
    h = hashlib.blake2b(("%d/%d/%d/%d" % (seed, kind, step, index)).encode(),
                        digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _torch_gen(device, seed: int, kind: int, step: int, index: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(seed, kind, step, index))
    return g


def torch_param(w: Workload, index: int, device, out=None):
    import torch
    spec = w.params[index]
    gen = _torch_gen(device, w.seed, KIND_PARAM, 0, index)
    t = out if out is not None else torch.empty(spec.shape, dtype=torch.float32, device=device)
    t.normal_(0.0, w.weight_std, generator=gen)
    return t


def torch_momentum(w: Workload, index: int, device, out=None):
    import torch
    spec = w.params[index]
    t = out if out is not None else torch.empty(spec.shape, dtype=torch.float32, device=device)
    if w.momentum_init_std == 0.0:
        t.zero_()
        return t
    gen = _torch_gen(device, w.seed, KIND_MOMENTUM, 0, index)
    t.normal_(0.0, w.momentum_init_std, generator=gen)
    return t


def torch_grad(w: Workload, step: int, index: int, device, out=None):
    import torch
    spec = w.params[index]
    gen = _torch_gen(device, w.seed, KIND_GRAD, step, index)
    t = out if out is not None else torch.empty(spec.shape, dtype=torch.float32, device=device)
    t.normal_(0.0, w.grad_std, generator=gen)
    if w.grad_row_scale is not None and len(spec.shape) >= 1:
        lo, hi = w.grad_row_scale
        s = torch.empty(spec.shape[0], dtype=torch.float32, device=device)
        s.uniform_(math.log(lo), math.log(hi), generator=gen).exp_()
        t.mul_(s.reshape((-1,) + (1,) * (len(spec.shape) - 1)))
    if w.spike is not None and len(spec.shape) == 2:
        rank, mag = w.spike
        m, n = spec.shape
        u = torch.randn((m, rank), generator=gen, device=device, dtype=torch.float32)
        v = torch.randn((rank, n), generator=gen, device=device, dtype=torch.float32)
        t.add_(torch.mm(u, v), alpha=mag / math.sqrt(rank))
    return t


MODE_IDS = {"muon_adamw": 0, "adamw": 1}   # the plan's optimizer modes


def mode_id(w: Workload) -> int:
    return MODE_IDS[w.mode]


def hparams_for(w: Workload) -> Dict[str, object]:
    """Hyperparameter overrides of a workload on top of the defaults
    (lr 2.5e-5, momentum 0.95 Nesterov, 5 NS steps, moonlight 0.2, AdamW
    betas (0.9, 0.999), eps 1e-8, decay 0.01, clip 1.0)."""
    return dict(w.hparams)


# --------------------------------------------------------------------------
# Gradients with a singular value decomposition known by construction
# --------------------------------------------------------------------------
#
# For matrices too large for any CPU check of the whole matrix: the canonical
# r x c gradient (r <= c) is G = U diag(sigma) V^T with U the orthonormal r x r
# DCT-II matrix and V^T a set of distinct rows of the orthonormal c x c one.
# Any product U diag(w) V^T of these factors then has rows that cost one
# length-c inverse DCT each.

KIND_SVD = 3


@dataclass(frozen=True)
class KnownSvd:
    r: int
    c: int
    sigma: np.ndarray    # (r,) float64, the singular values of G
    rows: np.ndarray     # (r,) int64, distinct rows of the c x c DCT matrix: V^T


def known_svd(seed: int, r: int, c: int, fro: float = 3.0,
              spread: Tuple[float, float] = (0.5, 1.5)) -> KnownSvd:
    """Singular values uniform in `spread`, scaled to Frobenius norm `fro`,
    and r distinct rows out of c, from one seeded stream."""
    if not 1 <= r <= c:
        raise ValueError("need 1 <= r <= c")
    g = _rng(seed, KIND_SVD, 0, 0)
    sigma = g.uniform(spread[0], spread[1], r)
    sigma *= fro / math.sqrt(float(np.dot(sigma, sigma)))
    rows = g.choice(c, size=r, replace=False).astype(np.int64)
    return KnownSvd(r, c, sigma, rows)


def dct_entries(n: int, k, j) -> np.ndarray:
    """Entries [k, j] (broadcast index arrays) of the orthonormal n x n DCT-II
    matrix, sqrt((1 or 2)/n) cos(pi (2j+1) k / (2n)), in float64; the angle is
    reduced exactly in integers first."""
    k = np.asarray(k, np.int64)
    j = np.asarray(j, np.int64)
    a = ((2 * j + 1) * k) % (4 * n)
    scale = np.where(k == 0, math.sqrt(1.0 / n), math.sqrt(2.0 / n))
    return scale * np.cos(np.pi * a.astype(np.float64) / (2 * n))


def np_known_svd_row(ks: KnownSvd, i: int, weights) -> np.ndarray:
    """Row i of U diag(weights) V^T (length c, float64)."""
    from scipy.fft import idct
    w = np.zeros(ks.c)
    w[ks.rows] = dct_entries(ks.r, i, np.arange(ks.r)) * np.asarray(weights, np.float64)
    return idct(w, type=2, norm="ortho")


def np_known_svd_matrix(ks: KnownSvd, weights) -> np.ndarray:
    """U diag(weights) V^T in full (small sizes only), float64."""
    r, c = ks.r, ks.c
    u = dct_entries(r, np.arange(r)[:, None], np.arange(r)[None, :])
    vt = dct_entries(c, ks.rows[:, None], np.arange(c)[None, :])
    return (u * np.asarray(weights, np.float64)) @ vt


def torch_known_svd_grad(ks: KnownSvd, device, transposed: bool = False, block: int = 2048):
    """G (or G^T when `transposed`) as float32 on `device`: formed in float64,
    rounded once.  V^T is built `block` rows at a time."""
    import torch
    r, c = ks.r, ks.c
    f64 = dict(dtype=torch.float64, device=device)
    i64 = dict(dtype=torch.int64, device=device)

    def dct(n, k, j):
        a = torch.remainder((2 * j + 1) * k, 4 * n).to(torch.float64)
        scale = torch.where(k == 0, torch.tensor(math.sqrt(1.0 / n), **f64),
                            torch.tensor(math.sqrt(2.0 / n), **f64))
        return scale * torch.cos(a * (math.pi / (2 * n)))

    ar = torch.arange(r, **i64)
    us = dct(r, ar[:, None], ar[None, :]) * torch.as_tensor(ks.sigma, **f64)[None, :]
    rows = torch.as_tensor(ks.rows, **i64)
    jc = torch.arange(c, **i64)
    g = torch.zeros((r, c), **f64)
    for k0 in range(0, r, block):
        k1 = min(r, k0 + block)
        vt = dct(c, rows[k0:k1, None], jc[None, :])
        g.addmm_(us[:, k0:k1].contiguous(), vt)
        del vt
    out = (g.t() if transposed else g).contiguous().to(torch.float32)
    del g, us
    return out
