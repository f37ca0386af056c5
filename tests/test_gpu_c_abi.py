"""The C ABI driven from plain C (tests/c/abi_step.c): no Python or torch in
the process that calls the library -- it allocates its own device buffers
with the HIP runtime, builds the plan, runs two steps on its own stream --
and its results match the CPU oracle to the same gates as the parity tests.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import _harness as H

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "abi_step")


def _table():
    return [W.ParamSpec("action_expert.layers.0.self_attn.q_proj.weight", (300, 300)),
            W.ParamSpec("action_expert.layers.0.mlp.up_proj.weight", (520, 130)),
            W.ParamSpec("action_expert.layers.0.mlp.down_proj.weight", (130, 520)),
            W.ParamSpec("vlm.model.layers.0.mlp.up_proj.weight", (96, 40)),
            W.ParamSpec("vlm.model.layers.0.input_layernorm.weight", (40,)),
            W.ParamSpec("vlm.model.norm.bias", (17,)),
            W.ParamSpec("vlm.model.embed_tokens.weight", (50, 40), trainable=False)]


@pytest.mark.parametrize("prec,overlap", [(0, 1), (1, 0)])
def test_plain_c_driver(tmp_path, prec, overlap):
    if not os.path.exists(EXE):
        pytest.fail("C driver not built: run python tests/c/build.py (build() does)")
    steps = 2
    w = W.Workload("c_abi", seed=11, steps=steps, ns_precision=("bf16", "fp32")[prec],
                   params=_table(), grad_std=1e-2)
    d = str(tmp_path)
    with open(os.path.join(d, "table.txt"), "w") as f:
        f.write("%d %d %d %d\n" % (len(w.params), steps, prec, overlap))
        for p in w.params:
            f.write("%s %d %d %s\n" % (p.name, int(p.trainable), len(p.shape),
                                       " ".join(str(s) for s in p.shape)))
    groups = O.route(w.names, w.shapes, w.trainable)
    params = [W.np_param(w, i) if groups[i] != O.NONE else None for i in range(len(w.params))]
    for i, p in enumerate(params):
        if p is not None:
            p.tofile(os.path.join(d, "param_%d.bin" % i))
    grads = {}
    for s in range(1, steps + 1):
        for i in range(len(w.params)):
            if groups[i] != O.NONE:
                grads[s, i] = W.np_grad(w, s, i)
                grads[s, i].tofile(os.path.join(d, "grad_%d_%d.bin" % (s, i)))
    H.say("C driver: %s prec=%d overlap=%d" % (EXE, prec, overlap))
    r = subprocess.run([EXE, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, "abi_step failed (%d): %s" % (r.returncode, r.stderr[-2000:])
    assert open(os.path.join(d, "out_status.txt")).read().startswith("ok")

    hp = O.HParams()
    n = len(w.params)
    zeros = [None if p is None else np.zeros_like(p) for p in params]
    p, buf, m, v = list(params), list(zeros), list(zeros), list(zeros)
    # moving average of |coef g|: the scale of m's rounding error (m may cancel)
    mabs = [None if z is None else z.astype(np.float64) for z in zeros]
    for s in range(1, steps + 1):
        res = O.optimizer_step(w.names, p, [grads.get((s, i)) for i in range(n)], w.trainable,
                               buf, m, v, s, hp, groups=groups)
        p, buf, m, v = res.params, res.muon_momentum, res.adam_m, res.adam_v
        for i in range(n):
            if groups[i] == O.ADAMW:
                mabs[i] = hp.beta1 * mabs[i] + (1 - hp.beta1) * np.abs(
                    res.clip_coef * grads[s, i].astype(np.float64))
    norm = float(open(os.path.join(d, "out_norm.txt")).read())
    assert abs(norm - res.grad_norm) <= 1e-5 * res.grad_norm
    tol = H.BF16_TOL if prec == 0 else H.FP32_TOL

    def out(name, i):
        return np.fromfile(os.path.join(d, "%s_%d.bin" % (name, i)), np.float32).reshape(
            w.params[i].shape)

    for i in range(n):
        if groups[i] == O.ADAMW:
            H.check_adamw(out("out_param", i), out("out_m", i), out("out_v", i),
                          p[i], m[i], v[i], "C driver entry %d" % i, m_terms=mabs[i])
        elif groups[i] == O.MUON:
            np.testing.assert_allclose(out("out_buf", i), buf[i], rtol=1e-5,
                                       atol=1e-7 * float(np.abs(buf[i]).max()))
            err = H.rel_fro(out("out_delta", i), res.deltas[i])
            assert err <= tol, "C driver entry %d: delta rel err %.3g" % (i, err)
