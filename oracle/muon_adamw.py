"""Plain, slow fp64 reference of the hybrid MuonAdamW optimizer step.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It is written for a
reader checking it against the OpenDM training-stack page by eye: one function
per step of the method, NumPy float64 arithmetic, matrix products through
NumPy's BLAS, no blocking, fusion or reordering.  Inputs and stored state are
float32 (the storage contract of the GPU library); every step computes in
float64 and rounds stored state back to float32 once, at the end of the step.

Citations name the page and the part of it a function follows:
  [routing]      Muon/AdamW hybrid section, "how parameters are split" table
                 (2-D, under action_expert ... layers, ends in .weight, with
                 embeddings and norms excluded; everything else goes to AdamW;
                 the optim switch muon_adamw / adamw)
  [NS]           Muon/AdamW hybrid section, Newton-Schulz paragraph
                 (a 5-step Newton-Schulz iteration approximates the zeroth
                 power of the matrix instead of an SVD)
  [hparams]      hyperparameter table of DM05OptimizerConfig (momentum 0.95,
                 Nesterov on, 5 NS steps, moonlight coefficient 0.2, base lr
                 2.5e-5) and the sentence after it giving the Muon learning rate
                 lr * muon_lr_scale * 0.2 * sqrt(max(shape))
  [FSDP-plan]    the MuonShardPlan paragraph: NS always acts on the whole
                 matrix, never on a shard
  [frozen]       FSDP section: the VLM token embedding and its tied lm_head are
                 frozen by default
  [defaults]     defaults quick-reference table (max_grad_norm 1.0; learning
                 rate schedule cosine_with_min_lr with min_lr_rate 0.1)
  [precision]    mixed-precision section: the default bf16_mixed policy
                 stores the model in bfloat16; fp32_mixed keeps fp32 weights

Readings where the page is silent (each also listed in the design notes):
  * NS quintic coefficients: the page gives none.  Default (3.2608, -3.6447,
    1.3650), a fixed triple whose 5-fold composition keeps every singular value
    of a Frobenius-normalised input with sigma/||X||_F in [1e-2, 1] inside
    [0.934, 1.215]; the widely published (3.4445, -4.7750, 2.0315) is accepted
    as an option.
  * Canonical orientation: rows <= cols, the Gram matrix is X X^T; a matrix
    stored with more rows than columns is transposed before NS and back after.
  * Normalisation epsilon 1e-7 added to the Frobenius norm.
  * Nesterov in sum form: buf = mu*buf + g ; u = g + mu*buf.
  * muon_lr_scale = 1.0; "shape" is the stored (m, n); the shape factor is
    computed in float64 and rounded once to float32.
  * Muon weight decay 0 unless given (then decoupled, scaled by the base lr).
  * AdamW is the decoupled-decay algorithm of torch.optim.AdamW with one step
    counter for the group; decay applies to every AdamW tensor.
  * Clipping is global over every trainable gradient of both groups, with the
    1e-6 guard of the usual clip_grad_norm_, and is applied before both
    updates; max_grad_norm <= 0 disables it; non-finite norms propagate.
  * The schedule cosine_with_min_lr is the half-cosine from the base lr down
    to min_lr_rate * lr over total_steps scheduler steps after a linear
    warmup from 0 (0 warmup steps unless given), as the HF-Trainer family's
    scheduler of that name computes it up to total_steps; the scheduler step
    of optimizer step t (counted from 1) is t - 1.  Past total_steps the rate
    stays at its minimum: this oracle's own reading (that scheduler would
    follow the cosine back up).  The schedule scales the lr of both groups.
  * bf16 parameter storage (bf16_mixed): parameters and their gradients are
    bfloat16 values; optimizer states (AdamW moments, Muon momentum) stay
    float32; the step computes as for fp32 storage and rounds the new
    parameter once to bfloat16, ties to even.  There is no float32 master
    copy, so an update smaller than half a bfloat16 spacing leaves the
    parameter unchanged.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "MUON", "ADAMW", "NONE", "GROUP_NAMES",
    "MODE_MUON_ADAMW", "MODE_ADAMW",
    "DEFAULT_NS_COEFFS", "PUBLISHED_NS_COEFFS",
    "HParams", "schedule_factor", "scheduled_lr",
    "route_one", "route", "lr_shape_scale", "plan_dump",
    "global_grad_norm", "clip_coefficient",
    "adamw_update", "nesterov_momentum", "frobenius_normalise",
    "newton_schulz", "ns_spectral_map", "newton_schulz_bf16_emulated", "ns_bf16_policy_iterate",
    "bf16_split", "bf16_round",
    "bf16_round_f64", "store_param",
    "muon_matrix_update", "optimizer_step",
]

MUON, ADAMW, NONE = 0, 1, 2
GROUP_NAMES = {MUON: "MUON", ADAMW: "ADAMW", NONE: "NONE"}
MODE_MUON_ADAMW, MODE_ADAMW = 0, 1

DEFAULT_NS_COEFFS = (3.2608, -3.6447, 1.3650)
PUBLISHED_NS_COEFFS = (3.4445, -4.7750, 2.0315)


@dataclass
class HParams:
    """Defaults from [hparams] and [defaults]; AdamW's betas, eps and decay
    are the ones stated for the tiny hybrid workload."""
    lr: float = 2.5e-5
    muon_lr_scale: float = 1.0
    muon_momentum: float = 0.95
    muon_nesterov: bool = True
    muon_ns_steps: int = 5
    ns_coeffs: Tuple[float, float, float] = DEFAULT_NS_COEFFS
    ns_eps: float = 1e-7
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    muon_weight_decay: float = 0.0
    max_grad_norm: float = 1.0
    moonlight_coefficient: float = 0.2
    lr_schedule: str = "constant"        # or "cosine_with_min_lr"  [defaults]
    warmup_steps: int = 0
    total_steps: int = 0
    min_lr_rate: float = 0.1
    # how parameters (and their gradients) are stored [precision]: "fp32",
    # or "bf16" for the bf16_mixed policy's bfloat16 model; optimizer states
    # stay float32 either way
    param_storage: str = "fp32"


def schedule_factor(hp: HParams, k: int) -> float:
    """Multiplier of the base lr at scheduler step k (0, 1, ...).  [defaults]

    constant: 1.  cosine_with_min_lr: k / warmup during the linear warmup;
    then, with progress p = (k - warmup) / (total - warmup) held at 1 past the
    end, min_lr_rate + (1 - min_lr_rate) * (1 + cos(pi p)) / 2, which runs
    from 1 down to min_lr_rate along half a cosine period."""
    if hp.lr_schedule == "constant":
        return 1.0
    if hp.lr_schedule != "cosine_with_min_lr":
        raise ValueError("unknown lr schedule %r" % (hp.lr_schedule,))
    warm, total = int(hp.warmup_steps), int(hp.total_steps)
    if k < warm:
        return k / max(1, warm)
    progress = min(1.0, (k - warm) / max(1, total - warm))
    half_cosine = 0.5 * (1.0 + math.cos(math.pi * progress))
    return hp.min_lr_rate + (1.0 - hp.min_lr_rate) * half_cosine


def scheduled_lr(hp: HParams, t: int) -> float:
    """Learning rate of optimizer step t (counted from 1)."""
    return hp.lr * schedule_factor(hp, t - 1)


# --------------------------------------------------------------------------
# Routing and the plan  [routing], [frozen], [hparams], [FSDP-plan]
# --------------------------------------------------------------------------

_EXCLUDED_SUBSTRINGS = ("embed", "lm_head", "norm")


def route_one(name: str, shape: Sequence[int], trainable: bool,
              mode: int = MODE_MUON_ADAMW) -> int:
    """Group of one parameter.  [routing]

    Frozen parameters take no update and no part in the clip norm ([frozen]:
    the routing scans trainable parameters only).  With the optim switch set
    to plain AdamW every trainable tensor is AdamW.  Otherwise a tensor is
    Muon when it is a matrix (two dimensions) whose dotted name contains
    'action_expert' in one component, has a component exactly 'layers' after
    that one, ends with '.weight', and whose name, with ASCII letters folded
    to lower case, contains none of 'embed', 'lm_head', 'norm' (the page's
    exclusion of embeddings and of every norm layer).  Anything else
    trainable is AdamW.
    """
    if not trainable:
        return NONE
    if mode == MODE_ADAMW:
        return ADAMW
    if len(shape) != 2:
        return ADAMW
    if not name.endswith(".weight"):
        return ADAMW
    parts = name.split(".")
    ae = None
    for i, part in enumerate(parts):
        if "action_expert" in part:
            ae = i
            break
    if ae is None:
        return ADAMW
    if "layers" not in parts[ae + 1:]:
        return ADAMW
    lowered = name.encode("utf-8").lower()      # ASCII case folding only
    for bad in _EXCLUDED_SUBSTRINGS:
        if bad.encode() in lowered:
            return ADAMW
    return MUON


def route(names: Sequence[str], shapes: Sequence[Sequence[int]],
          trainable: Sequence[bool], mode: int = MODE_MUON_ADAMW) -> List[int]:
    return [route_one(n, s, t, mode) for n, s, t in zip(names, shapes, trainable)]


def lr_shape_scale(m: int, n: int, moonlight_coefficient: float = 0.2) -> np.float32:
    """The shape factor moonlight_coefficient * sqrt(max(m, n)) of the Muon
    learning rate, in float64, rounded once to float32.  [hparams]"""
    return np.float32(moonlight_coefficient * math.sqrt(float(max(m, n))))


def _f32_bits(x: np.float32) -> str:
    return "%08x" % int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def plan_dump(names: Sequence[str], shapes: Sequence[Sequence[int]],
              trainable: Sequence[bool], mode: int = MODE_MUON_ADAMW,
              moonlight_coefficient: float = 0.2) -> str:
    """Canonical text of a plan: the routing of every entry, the stored and
    canonical (rows <= cols) shape of every Muon matrix, its orientation flag,
    its shape-bucket (distinct canonical shapes, numbered in order of first
    appearance), the bits of its float32 shape factor, and the running offset
    of every AdamW tensor in the concatenated AdamW element space.

    This format is an interface: the library's plan dump must produce the
    same bytes for the same table.
    """
    groups = route(names, shapes, trainable, mode)
    buckets: Dict[Tuple[int, int], int] = {}
    bucket_count: Dict[int, int] = {}
    lines = []
    adam_off = 0
    n_m = n_a = n_n = 0
    for i, (name, shape, g) in enumerate(zip(names, shapes, groups)):
        numel = 1
        for d in shape:
            numel *= int(d)
        if g == MUON:
            n_m += 1
            m, n = int(shape[0]), int(shape[1])
            r, c = min(m, n), max(m, n)
            if (r, c) not in buckets:
                buckets[(r, c)] = len(buckets)
            b = buckets[(r, c)]
            bucket_count[b] = bucket_count.get(b, 0) + 1
            lines.append("%d MUON %d %d %d %d %d %d %s %d -1" % (
                i, b, m, n, r, c, 1 if m > n else 0,
                _f32_bits(lr_shape_scale(m, n, moonlight_coefficient)), numel))
        elif g == ADAMW:
            n_a += 1
            lines.append("%d ADAMW -1 0 0 0 0 0 00000000 %d %d" % (i, numel, adam_off))
            adam_off += numel
        else:
            n_n += 1
            lines.append("%d NONE -1 0 0 0 0 0 00000000 %d -1" % (i, numel))
    head = ["muon_adamw_plan v1 mode=%d entries=%d muon=%d adamw=%d none=%d "
            "buckets=%d adamw_numel=%d" % (mode, len(groups), n_m, n_a, n_n,
                                          len(buckets), adam_off)]
    for (r, c), b in sorted(buckets.items(), key=lambda kv: kv[1]):
        head.append("bucket %d r=%d c=%d count=%d" % (b, r, c, bucket_count[b]))
    return "\n".join(head + lines) + "\n"


# --------------------------------------------------------------------------
# Global gradient-norm clipping  [defaults]
# --------------------------------------------------------------------------

def global_grad_norm(grads: Sequence[np.ndarray]) -> float:
    """sqrt of the sum of squares of every element of every given gradient,
    accumulated in float64."""
    total = 0.0
    for g in grads:
        g64 = np.asarray(g, dtype=np.float64).ravel()
        total += float(np.dot(g64, g64))
    return math.sqrt(total)


def clip_coefficient(norm: float, max_grad_norm: float) -> float:
    """Factor applied to every gradient before the update: 1 when clipping is
    off (max_grad_norm <= 0), else min(1, max_grad_norm / (norm + 1e-6)),
    clamped like a tensor clamp: a NaN norm gives a NaN factor."""
    if max_grad_norm <= 0.0:
        return 1.0
    coef = max_grad_norm / (norm + 1e-6)
    if math.isnan(coef):
        return coef                     # a NaN norm poisons every update
    return min(1.0, coef)


# --------------------------------------------------------------------------
# AdamW group  [routing] (tensors not selected for Muon go to AdamW)
# --------------------------------------------------------------------------

def adamw_update(p, g, m, v, t: int, coef: float, hp: HParams):
    """One decoupled-weight-decay Adam step (the AdamW of torch.optim), in
    float64, on arrays of any shape.  t is the 1-based step count.

    g' = coef*g
    p  = p*(1 - lr*wd)
    m  = beta1*m + (1-beta1)*g'
    v  = beta2*v + (1-beta2)*g'^2
    p  = p - (lr / (1-beta1^t)) * m / (sqrt(v)/sqrt(1-beta2^t) + eps)

    Returns (p as stored under hp.param_storage, m float32, v float32).
    """
    p = np.asarray(p, np.float64)
    g = np.asarray(g, np.float64) * coef
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    bc1 = 1.0 - hp.beta1 ** t
    bc2 = 1.0 - hp.beta2 ** t
    p = p * (1.0 - hp.lr * hp.weight_decay)
    m = hp.beta1 * m + (1.0 - hp.beta1) * g
    v = hp.beta2 * v + (1.0 - hp.beta2) * g * g
    denom = np.sqrt(v) / math.sqrt(bc2) + hp.eps
    p = p - (hp.lr / bc1) * m / denom
    return store_param(p, hp.param_storage), m.astype(np.float32), v.astype(np.float32)


# --------------------------------------------------------------------------
# Muon group  [hparams], [NS], [FSDP-plan]
# --------------------------------------------------------------------------

def nesterov_momentum(g, buf, coef: float, mu: float, nesterov: bool):
    """Momentum with coefficient mu on the clipped gradient; with Nesterov on,
    the direction looks one step ahead along the new buffer.

    buf = mu*buf + coef*g
    u   = coef*g + mu*buf   (Nesterov)   or   u = buf

    Returns (u float64, new buf float64)."""
    g = np.asarray(g, np.float64) * coef
    buf = mu * np.asarray(buf, np.float64) + g
    u = g + mu * buf if nesterov else buf
    return u, buf


def frobenius_normalise(x, eps: float):
    """x / (||x||_F + eps)."""
    x = np.asarray(x, np.float64)
    return x / (math.sqrt(float(np.sum(x * x))) + eps)


def newton_schulz(u, steps: int, coeffs=DEFAULT_NS_COEFFS, eps: float = 1e-7):
    """Quintic Newton-Schulz iteration towards the orthogonal polar factor of
    the whole matrix u (the 'zeroth power' of [NS]), in float64.

    The matrix is put in the orientation with rows <= columns, so the Gram
    matrix X X^T is the smaller square; it is scaled to unit Frobenius norm;
    then each step is
        A = X X^T ;  B = b*A + c*(A A) ;  X = a*X + B X
    and the result is turned back to the input's orientation.
    """
    u = np.asarray(u, np.float64)
    if u.ndim != 2:
        raise ValueError("newton_schulz needs a matrix")
    a, b, c = (float(v) for v in coeffs)
    tall = u.shape[0] > u.shape[1]
    x = u.T if tall else u
    x = frobenius_normalise(x, eps)
    for _ in range(steps):
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x.T if tall else x


def ns_spectral_map(s, steps: int, coeffs=DEFAULT_NS_COEFFS) -> np.ndarray:
    """What the NS iteration does to each singular value of its normalised
    input [NS]: for X = U diag(s) V^T, A = X X^T = U diag(s^2) U^T, so one
    step gives U diag(a s + b s^3 + c s^5) V^T; `steps` steps compose that
    scalar map.  For inputs whose SVD is known by construction, at sizes the
    matrix iteration cannot reach on a CPU."""
    s = np.asarray(s, np.float64)
    a, b, c = (float(v) for v in coeffs)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def bf16_round_f64(x) -> np.ndarray:
    """Round float64 values directly to the nearest bfloat16 (ties to even),
    returned as float32: no intermediate float32 rounding, which could move
    a value onto a tie.  bfloat16 has 8 significant bits and float32's
    exponent range (subnormals spaced 2^-133); beyond its largest value the
    result is infinite."""
    x = np.asarray(x, np.float64)
    shape = x.shape
    x = np.ascontiguousarray(x).ravel()
    bits = x.view(np.uint64)
    drop = np.uint64(52 - 7)                       # float64 mantissa bits below bf16's
    lsb = (bits >> drop) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    rounded = ((bits + half + lsb) & ~np.uint64((1 << 45) - 1)).view(np.float64)
    tiny = np.abs(x) < 2.0 ** -126                  # bf16 subnormal range: fixed spacing
    if np.any(tiny):
        q = 2.0 ** -133
        rounded = np.where(tiny, np.rint(x / q) * q, rounded)   # rint: ties to even
    rounded = np.where(np.isnan(x), np.nan, rounded)
    with np.errstate(over="ignore"):
        out = rounded.astype(np.float32)
    return out.reshape(shape)


def store_param(p, storage: str) -> np.ndarray:
    """A float64 parameter value as stored [precision]: rounded once to
    float32, or to bfloat16 (ties to even) under bf16 storage."""
    if storage == "fp32":
        return np.asarray(p, np.float64).astype(np.float32)
    if storage == "bf16":
        return bf16_round_f64(p)
    raise ValueError("unknown parameter storage %r" % (storage,))


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32.  Diagnostic helper for the bf16-emulating NS below."""
    f = np.ascontiguousarray(np.asarray(x, np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    nan = np.isnan(f)
    out = rounded.view(np.float32).copy()
    out[nan] = np.nan
    return out.reshape(f.shape)


def bf16_split(x):
    """A float32 value as a pair of bfloat16 values: hi = bf16(x) and
    lo = bf16(x - hi), so hi + lo holds 16 significant bits of x (x - hi is
    exact in float32).  Returned as float64 arrays."""
    x = np.asarray(x, np.float32)
    hi = bf16_round(x)
    lo = bf16_round(x - hi)
    return hi.astype(np.float64), lo.astype(np.float64)


def _f32(x) -> np.ndarray:
    """float64 values rounded once to float32, returned as float64 (the
    float32 accumulators of a product, modelled as exact sums rounded
    once)."""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def ns_bf16_policy_iterate(x0, steps: int, coeffs=DEFAULT_NS_COEFFS, lo_iters=None):
    """Diagnostic model of a bfloat16 precision policy for the NS iteration
    [NS] (not a parity target; the pages fix no precision for it).  x0 is the
    normalised input in rows <= cols orientation, as float32.

    The master X is a bf16 pair (hi, lo) (bf16_split).  Each step:
        A   = bf16(f32(hi hi^T))                 Gram of the bf16 operand
        B   = bf16(f32(b A + c f32(A A)))        the same bf16 A in both terms
        Y   = f32(a (hi + lo) + f32(B hi))       linear term from the pair
        (hi, lo) = bf16_split(Y)
    and the result is the last Y (float32).  Steps numbered lo_iters and
    later (default: none) take the linear term from hi alone, so the lo half
    is neither needed nor kept for them.  f32(.) is a float64 value rounded
    once to float32; bf16(.) rounds float32 to bfloat16, ties to even."""
    a, b, c = (float(v) for v in coeffs)
    lo_iters = steps if lo_iters is None else int(lo_iters)
    hi, lo = bf16_split(x0)
    y = np.asarray(x0, np.float64)
    for k in range(steps):
        gram = bf16_round(_f32(hi @ hi.T)).astype(np.float64)
        poly = bf16_round(_f32(b * gram + c * _f32(gram @ gram))).astype(np.float64)
        lin = hi + lo if k < lo_iters else hi
        y = _f32(a * lin + _f32(poly @ hi))
        if k + 1 < steps:
            hi, lo = bf16_split(y)
    return y


def newton_schulz_bf16_emulated(u, steps: int, coeffs=DEFAULT_NS_COEFFS,
                                eps: float = 1e-7, lo_iters=None):
    """Diagnostic only, not a parity target: newton_schulz with its products
    taken under the bf16 policy of ns_bf16_policy_iterate (orientation and
    normalisation as in newton_schulz, the normalised input rounded once to
    float32).  It tells how much of a bf16 GPU result's distance from
    `newton_schulz` is inherent to that policy."""
    u = np.asarray(u, np.float64)
    tall = u.shape[0] > u.shape[1]
    x = (u.T if tall else u)
    x0 = frobenius_normalise(x, eps).astype(np.float32)
    y = ns_bf16_policy_iterate(x0, steps, coeffs, lo_iters)
    return y.T if tall else y


def muon_matrix_update(p, g, buf, coef: float, hp: HParams, shape_scale):
    """The whole Muon update of one matrix parameter (float64 inside).

    u, buf = nesterov_momentum(...)            [hparams]
    O      = newton_schulz(u, ns_steps)        [NS], on the full matrix [FSDP-plan]
    delta  = lr * muon_lr_scale * shape_scale * O   [hparams]
    p      = p*(1 - lr*muon_wd) - delta

    Returns (p as stored under hp.param_storage, buf float32, delta float64)."""
    u, buf = nesterov_momentum(g, buf, coef, hp.muon_momentum, hp.muon_nesterov)
    o = newton_schulz(u, hp.muon_ns_steps, hp.ns_coeffs, hp.ns_eps)
    lr_eff = float(hp.lr) * float(hp.muon_lr_scale) * float(shape_scale)
    delta = lr_eff * o
    p = np.asarray(p, np.float64) * (1.0 - hp.lr * hp.muon_weight_decay) - delta
    return store_param(p, hp.param_storage), buf.astype(np.float32), delta


@dataclass
class StepResult:
    params: List[Optional[np.ndarray]]
    muon_momentum: List[Optional[np.ndarray]]
    adam_m: List[Optional[np.ndarray]]
    adam_v: List[Optional[np.ndarray]]
    deltas: List[Optional[np.ndarray]]
    grad_norm: float
    clip_coef: float
    groups: List[int] = field(default_factory=list)


def optimizer_step(names, params, grads, trainable, muon_momentum, adam_m,
                   adam_v, t: int, hp: HParams, mode: int = MODE_MUON_ADAMW,
                   groups: Optional[Sequence[int]] = None) -> StepResult:
    """One hybrid step over a whole parameter table, in the page's order:
    route (once), clip over all trainable gradients, then AdamW for the AdamW
    group and momentum -> NS -> scaled update for the Muon group.

    params/grads/state are lists indexed like `names` (None where unused).
    Nothing is modified in place; new float32 arrays are returned."""
    shapes = [np.shape(p) if p is not None else np.shape(g) for p, g in zip(params, grads)]
    if groups is None:
        groups = route(names, shapes, trainable, mode)
    # the schedule sets this step's lr for both groups
    hp = replace(hp, lr=scheduled_lr(hp, t))
    live = [g for g, grp in zip(grads, groups) if grp != NONE]
    norm = global_grad_norm(live)
    coef = clip_coefficient(norm, hp.max_grad_norm)
    n = len(names)
    out_p: List[Optional[np.ndarray]] = [None] * n
    out_buf: List[Optional[np.ndarray]] = [None] * n
    out_m: List[Optional[np.ndarray]] = [None] * n
    out_v: List[Optional[np.ndarray]] = [None] * n
    deltas: List[Optional[np.ndarray]] = [None] * n
    for i in range(n):
        grp = groups[i]
        if grp == ADAMW:
            out_p[i], out_m[i], out_v[i] = adamw_update(
                params[i], grads[i], adam_m[i], adam_v[i], t, coef, hp)
        elif grp == MUON:
            m, nn = shapes[i]
            scale = lr_shape_scale(m, nn, hp.moonlight_coefficient)
            out_p[i], out_buf[i], deltas[i] = muon_matrix_update(
                params[i], grads[i], muon_momentum[i], coef, hp, scale)
        else:
            out_p[i] = None if params[i] is None else np.asarray(params[i], np.float32).copy()
    return StepResult(out_p, out_buf, out_m, out_v, deltas, norm, coef, list(groups))
