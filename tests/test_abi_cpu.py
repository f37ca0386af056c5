"""Host-side tests of the C-ABI library (no GPU needed).

* the built library loads and exports every function include/muon_adamw.h
  declares;
* the plan (routing, canonical shapes, buckets, shape factors, AdamW offsets)
  matches the oracle's plan dump byte for byte on every synthetic workload and
  on the adversarial routing table;
* every argument error is reported before anything is launched (pointers
  passed here are never dereferenced: validation fails first).
"""

import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_adamw.h")

M = pytest.importorskip("muon_newton_schulz_02_amd")


@pytest.fixture(scope="module")
def lib():
    try:
        return M.load_library()
    except RuntimeError as e:
        pytest.fail("library not built: %s" % e)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_adamw_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) == 12, names
    for n in names:
        assert hasattr(lib, n), n
    from muon_newton_schulz_02_amd import _abi
    assert sorted(s[0] for s in _abi.SIGNATURES) == names


def test_version_and_defaults(lib):
    assert "gfx950" in M.muon_adamw_version()
    hp = M.muon_adamw_default_hparams()
    assert hp.lr == 2.5e-5
    assert hp.muon_momentum == 0.95 and hp.muon_nesterov == 1
    assert hp.muon_ns_steps == 5 and hp.max_grad_norm == 1.0
    assert tuple(hp.ns_coeffs) == O.DEFAULT_NS_COEFFS
    assert hp.ns_precision == M.MA_NS_BF16
    assert hp.lr_schedule == M.MA_LR_CONSTANT and hp.min_lr_rate == 0.1
    assert hp.warmup_steps == 0 and hp.total_steps == 0


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_plan_dump_matches_oracle(lib, name):
    w = W.WORKLOADS[name]()
    plan = M.muon_adamw_plan(list(zip(w.names, w.shapes, w.trainable)), mode=W.mode_id(w))
    assert M.muon_adamw_plan_dump(plan) == O.plan_dump(w.names, w.shapes, w.trainable,
                                                       mode=W.mode_id(w))
    assert M.muon_adamw_plan_size(plan) == len(w.names)


def _golden_routing():
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "routing_table.txt")):
        if line.startswith("#") or not line.strip():
            continue
        grp, tr, shape, name = line.rstrip("\n").split("\t")
        rows.append((name, tuple(int(s) for s in shape.split(",")), tr == "1"))
    return rows


@pytest.mark.parametrize("mode", [O.MODE_MUON_ADAMW, O.MODE_ADAMW])
@pytest.mark.parametrize("moon", [0.2, 0.37])
def test_plan_dump_adversarial(lib, mode, moon):
    rows = _golden_routing()
    names, shapes, tr = zip(*rows)
    plan = M.muon_adamw_plan(rows, mode=mode, moonlight_coefficient=moon)
    assert M.muon_adamw_plan_dump(plan) == O.plan_dump(names, shapes, tr, mode, moon)


def test_plan_entries_and_shape_scale_bits(lib):
    rng = np.random.default_rng(0)
    table = []
    for i in range(200):
        m, n = (int(x) for x in rng.integers(1, 20000, 2))
        table.append(("action_expert.layers.%d.w.weight" % i, (m, n), True))
    plan = M.muon_adamw_plan(table)
    for i, (_, (m, n), _) in enumerate(table):
        e = M.muon_adamw_plan_entry(plan, i)
        assert e["group"] == M.MA_GROUP_MUON
        assert (e["m"], e["n"], e["r"], e["c"]) == (m, n, min(m, n), max(m, n))
        assert e["transposed"] == (1 if m > n else 0)
        assert np.float32(e["lr_shape_scale"]) == O.lr_shape_scale(m, n)
    names, shapes, tr = zip(*table)
    assert M.muon_adamw_plan_dump(plan) == O.plan_dump(names, shapes, tr)


def test_plan_errors(lib):
    with pytest.raises(M.MuonAdamWError) as e:
        M.muon_adamw_plan([])
    assert e.value.code == M.MA_ERR_INVALID_ARG
    with pytest.raises(M.MuonAdamWError) as e:
        M.muon_adamw_plan([("a.weight", (3, 0), True)])
    assert e.value.code == M.MA_ERR_SHAPE
    with pytest.raises(M.MuonAdamWError) as e:
        M.muon_adamw_plan([("a.weight", (1,) * 9, True)])
    assert e.value.code == M.MA_ERR_UNSUPPORTED
    with pytest.raises(M.MuonAdamWError) as e:
        M.muon_adamw_plan([("a.weight", (4, 4), True)], mode=7)
    assert e.value.code == M.MA_ERR_INVALID_ARG
    with pytest.raises(M.MuonAdamWError) as e:
        M.muon_adamw_plan([("a.weight", (4, 4), True)], moonlight_coefficient=-1.0)
    assert e.value.code == M.MA_ERR_INVALID_ARG
    with pytest.raises(M.MuonAdamWError) as e:
        M.muon_adamw_plan([("a.weight", (1 << 40, 1 << 40), True)])
    assert e.value.code == M.MA_ERR_SHAPE
    # a Muon matrix whose padded fp32 operand would pass 2 GiB (the 32-bit
    # buffer offsets of the GEMM loaders) is refused; the same shape routed to
    # AdamW, and the largest Muon matrix that fits, are accepted
    big = "action_expert.layers.0.q.weight"
    with pytest.raises(M.MuonAdamWError) as e:
        M.muon_adamw_plan([(big, (16384, 32768 + 1), True)])
    assert e.value.code == M.MA_ERR_SHAPE and "too large" in M.muon_adamw_last_error()
    M.muon_adamw_plan([("vlm.big.weight", (16384, 32769), True)])
    M.muon_adamw_plan([(big, (16384, 32768 - 256), True)])
    plan = M.muon_adamw_plan([("a.weight", (4, 4), True)])
    with pytest.raises(M.MuonAdamWError):
        M.muon_adamw_plan_entry(plan, 5)
    with pytest.raises(M.MuonAdamWError):
        M.muon_adamw_workspace_size(plan, 9)
    assert "range" in M.muon_adamw_last_error() or "precision" in M.muon_adamw_last_error()


def test_plan_dump_small_buffer(lib):
    from muon_newton_schulz_02_amd import _abi
    plan = M.muon_adamw_plan([("action_expert.layers.0.q.weight", (8, 4), True)])
    n = C.c_size_t()
    buf = C.create_string_buffer(4)
    rc = _abi.load().muon_adamw_plan_dump(plan.handle, buf, 4, C.byref(n))
    assert rc == M.MA_ERR_WORKSPACE and n.value > 4


def _table_small():
    return [("action_expert.layers.0.q.weight", (8, 4), True),
            ("vlm.model.norm.weight", (16,), True),
            ("vlm.model.embed_tokens.weight", (10, 4), False)]


def test_step_argument_errors_launch_nothing(lib):
    """Validation fails before any HIP call, so fake addresses are safe."""
    plan = M.muon_adamw_plan(_table_small())
    ws_need = M.muon_adamw_workspace_size(plan, M.MA_NS_BF16)
    fake = 1 << 40
    st = M.State(3)
    st.muon_momentum[0] = fake
    st.adam_m[1] = fake
    st.adam_v[1] = fake
    params = [fake, fake, None]
    grads = [fake, fake, None]

    def run(hp=None, ws=(fake, ws_need), params=params, grads=grads, state=st):
        hp = hp or M.muon_adamw_default_hparams()
        with pytest.raises(M.MuonAdamWError) as e:
            M.muon_adamw_step(plan, params, grads, state, hp, ws, stream=0)
        return e.value.code

    assert run(ws=(fake, ws_need - 1)) == M.MA_ERR_WORKSPACE
    assert run(ws=(fake + 4, ws_need)) == M.MA_ERR_WORKSPACE
    assert run(ws=(0, ws_need)) == M.MA_ERR_WORKSPACE
    assert run(hp=M.muon_adamw_default_hparams(muon_ns_steps=0)) == M.MA_ERR_UNSUPPORTED
    assert run(hp=M.muon_adamw_default_hparams(ns_precision=3)) == M.MA_ERR_UNSUPPORTED
    assert run(hp=M.muon_adamw_default_hparams(lr=float("nan"))) == M.MA_ERR_INVALID_ARG
    assert run(hp=M.muon_adamw_default_hparams(beta1=1.0)) == M.MA_ERR_INVALID_ARG
    cos = dict(lr_schedule="cosine_with_min_lr")
    assert run(hp=M.muon_adamw_default_hparams(lr_schedule=7)) == M.MA_ERR_INVALID_ARG
    assert run(hp=M.muon_adamw_default_hparams(total_steps=0, **cos)) == M.MA_ERR_INVALID_ARG
    assert run(hp=M.muon_adamw_default_hparams(total_steps=5, warmup_steps=6, **cos)) == \
        M.MA_ERR_INVALID_ARG
    assert run(hp=M.muon_adamw_default_hparams(total_steps=5, warmup_steps=-1, **cos)) == \
        M.MA_ERR_INVALID_ARG
    assert run(hp=M.muon_adamw_default_hparams(total_steps=5, min_lr_rate=1.5, **cos)) == \
        M.MA_ERR_INVALID_ARG
    assert run(params=[fake, None, None]) == M.MA_ERR_INVALID_ARG
    assert run(grads=[None, fake, None]) == M.MA_ERR_INVALID_ARG
    st2 = M.State(3)
    st2.adam_m[1] = fake
    st2.adam_v[1] = fake
    assert run(state=st2) == M.MA_ERR_INVALID_ARG
    st3 = M.State(3)
    st3.muon_momentum[0] = fake
    st3.adam_m[1] = fake
    assert run(state=st3) == M.MA_ERR_INVALID_ARG
    assert st.step == 0


def test_step_refuses_overlapping_buffers(lib):
    """Aliased buffers (a parameter passed again as its gradient, moments
    that share memory, a workspace over a tensor) are refused from the
    pointers alone, before any HIP call; only overlapping cases are tried
    here, since a disjoint set would go on to launch."""
    plan = M.muon_adamw_plan(_table_small())
    ws_need = M.muon_adamw_workspace_size(plan, M.MA_NS_BF16)
    n0 = M.muon_adamw_plan_entry(plan, 0)["m"] * M.muon_adamw_plan_entry(plan, 0)["n"]
    base = 1 << 40
    gap = 1 << 30

    def addr(k):
        return base + k * gap

    def run(params, grads, mom, am, av, ws):
        st = M.State(3)
        st.muon_momentum[0] = mom
        st.adam_m[1] = am
        st.adam_v[1] = av
        with pytest.raises(M.MuonAdamWError) as e:
            M.muon_adamw_step(plan, params, grads, st, M.muon_adamw_default_hparams(),
                              (ws, ws_need), stream=0)
        assert st.step == 0
        return e.value.code, M.muon_adamw_last_error()

    ok = dict(params=[addr(0), addr(1), None], grads=[addr(2), addr(3), None],
              mom=addr(4), am=addr(5), av=addr(6), ws=addr(7))

    code, msg = run(**dict(ok, grads=[addr(0), addr(3), None]))
    assert code == M.MA_ERR_INVALID_ARG and "overlaps" in msg
    # the momentum starts in the last float of the Muon parameter
    code, msg = run(**dict(ok, mom=addr(0) + 4 * (n0 - 1)))
    assert code == M.MA_ERR_INVALID_ARG and "momentum" in msg
    code, _ = run(**dict(ok, av=addr(5) + 4))
    assert code == M.MA_ERR_INVALID_ARG
    code, _ = run(**dict(ok, ws=addr(1) - 256))
    assert code == M.MA_ERR_INVALID_ARG


def test_workspace_size_grows_with_precision(lib):
    w = W.ae18_muon_bf16()
    plan = M.muon_adamw_plan(list(zip(w.names, w.shapes, w.trainable)))
    b = M.muon_adamw_workspace_size(plan, M.MA_NS_BF16)
    f = M.muon_adamw_workspace_size(plan, M.MA_NS_FP32)
    # bf16: X hi/lo pairs, ping-pong (8 B per element) + A + B;
    # fp32: X + two X^T (12 B per element) + A + B
    rc = sum(min(s) * max(s) for s in w.shapes)
    assert b >= rc * 8 and f >= rc * 12
    assert f > b


def _header_defines():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(MA_\w+)\s+\(?(-?\d+)\)?", text)}


def test_binding_constants_match_header():
    from muon_newton_schulz_02_amd import _abi
    defs = _header_defines()
    assert "MA_ERR_CAPTURE" in defs and "MA_PROFILE_EVENTS" in defs
    for k, v in defs.items():
        assert getattr(_abi, k) == v, k


def test_binding_structs_match_header(tmp_path):
    """sizeof and every field offset of the public structs, as the C compiler
    lays them out from the header, equal the ctypes mirrors'."""
    import shutil
    import subprocess
    from muon_newton_schulz_02_amd import _abi
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = [_abi.ma_param_desc, _abi.ma_plan_opts, _abi.ma_plan_entry, _abi.ma_state,
               _abi.ma_hparams]
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "muon_adamw.h"',
             "int main(void) {"]
    for s in structs:
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (s.__name__, s.__name__))
        for f in s._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (
                s.__name__, f[0], s.__name__, f[0]))
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = dict(l.split() for l in subprocess.run([str(exe)], check=True, capture_output=True,
                                                 text=True).stdout.splitlines())
    for s in structs:
        assert int(out[s.__name__]) == C.sizeof(s), s.__name__
        for f in s._fields_:
            key = "%s.%s" % (s.__name__, f[0])
            assert int(out[key]) == getattr(s, f[0]).offset, key


def test_plan_param_dtype(lib):
    table = [("action_expert.layers.0.q.weight", (8, 8), True)]
    for dt in ("fp32", "bf16", M.MA_PARAM_FP32, M.MA_PARAM_BF16):
        M.muon_adamw_plan(table, param_dtype=dt)
    with pytest.raises(M.MuonAdamWError) as e:
        M.muon_adamw_plan(table, param_dtype=2)
    assert e.value.code == M.MA_ERR_INVALID_ARG


def test_binding_rejects_wrong_tensors(lib):
    """The binding checks dtype, layout and device before any call: a CPU
    tensor, a non-contiguous view, a float16 tensor and, for a bf16 plan, a
    float32 parameter are refused."""
    torch = pytest.importorskip("torch")
    plan = M.muon_adamw_plan([("vlm.w", (4, 4), True)])
    st = M.State(1)
    st.adam_m[0] = 1 << 40
    st.adam_v[0] = 1 << 40
    hp = M.muon_adamw_default_hparams()
    ws = (1 << 40, M.muon_adamw_workspace_size(plan, 0))
    cpu = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        M.muon_adamw_step(plan, [cpu], [cpu], st, hp, ws, stream=0)
    with pytest.raises(ValueError):
        M.muon_adamw_step(plan, [torch.zeros(4, 8)[:, :4]], [1 << 40], st, hp, ws, stream=0)
    with pytest.raises(TypeError):
        M.muon_adamw_step(plan, [torch.zeros(4, 4, dtype=torch.float16)], [1 << 40], st, hp, ws,
                          stream=0)
    bplan = M.muon_adamw_plan([("vlm.w", (4, 4), True)], param_dtype="bf16")
    with pytest.raises(TypeError):
        M.muon_adamw_step(bplan, [torch.zeros(4, 4)], [1 << 40], st, hp, ws, stream=0)
    with pytest.raises(TypeError):
        st.device_step = torch.zeros(1, dtype=torch.int32)
        M.muon_adamw_step(plan, [1 << 40], [1 << 40], st, hp, ws, stream=0)


def test_binding_checks_sizes_against_the_plan(lib):
    """Every tensor the binding passes is compared with its plan entry's
    element count (and the workspace with the plan's workspace size) before
    the library is called: a mis-sized parameter, gradient, state or update
    output, a list with more items than entries, or a short workspace is
    refused (here on CPU tensors: the size check comes before the device
    check)."""
    torch = pytest.importorskip("torch")
    plan = M.muon_adamw_plan([("action_expert.layers.0.q.weight", (4, 6), True),
                              ("vlm.b", (5,), True)])
    hp = M.muon_adamw_default_hparams()
    need = M.muon_adamw_workspace_size(plan, hp.ns_precision)
    ws = (1 << 40, need)
    A = 1 << 40

    def state(mom=A, m=A, v=A):
        st = M.State(2)
        st.muon_momentum[0] = mom
        st.adam_m[1] = m
        st.adam_v[1] = v
        return st

    def refused(params, grads, st=None, workspace=ws, upd=None, norm=None):
        with pytest.raises(ValueError, match="plan"):
            M.muon_adamw_step(plan, params, grads, st or state(), hp, workspace, stream=0,
                              grad_norm_out=norm, muon_update_out=upd)

    refused([torch.zeros(4, 5), A], [A, A])                     # 20 elements for 24
    refused([A, torch.zeros(6)], [A, A])                        # entry 1: 6 for 5
    refused([A, A], [A, torch.zeros(4, 6)])                      # entries swapped
    refused([A, A], [A, A], st=state(mom=torch.zeros(4, 7)))
    refused([A, A], [A, A], st=state(v=torch.zeros(4)))
    refused([A, A], [A, A], upd=[torch.zeros(3, 6), None])
    refused([A, A, A], [A, A])                                   # three items, two entries
    refused([A, A], [A, A], workspace=torch.zeros(need - 1, dtype=torch.uint8))
    refused([A, A], [A, A], norm=torch.zeros(0))
    refused([torch.zeros(4 * 6 * 4 - 1, dtype=torch.uint8), A], [A, A])   # raw bytes too few
    # the right sizes get as far as the device check
    with pytest.raises(ValueError, match="GPU"):
        M.muon_adamw_step(plan, [torch.zeros(4, 6), A], [A, A], state(), hp, ws, stream=0)


def test_noalloc_refuses_plans_beyond_its_scratch(lib):
    """The allocation-free step accepts plans whose workspace fits its
    per-device scratch and refuses larger ones before any GPU call
    (fake addresses are never dereferenced)."""
    from muon_newton_schulz_02_amd import _abi
    text = open(HEADER).read()
    assert "#define MA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert _abi.MA_NOALLOC_SCRATCH_BYTES == 64 << 20
    plan = M.muon_adamw_plan([("action_expert.layers.0.q.weight", (4096, 4096), True)])
    assert M.muon_adamw_workspace_size(plan, M.MA_NS_BF16) > M.MA_NOALLOC_SCRATCH_BYTES
    st = M.State(1)
    st.muon_momentum[0] = 1 << 40
    with pytest.raises(M.MuonAdamWError) as e:
        M.muon_adamw_step_noalloc(plan, [1 << 40], [1 << 41], st, M.muon_adamw_default_hparams())
    assert e.value.code == M.MA_ERR_WORKSPACE
    assert "scratch" in str(e.value)
    assert st.step == 0
