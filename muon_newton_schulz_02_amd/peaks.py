"""Ceilings of this GPU, measured by the hand-written probes of
libma_peaks.so (csrc/peaks.hip) in the calling process: the matrix-core
issue rate (bf16 and fp32 MFMA, with the shader clock they ran at), the LDS
read bandwidth per compute unit, HBM streams (read only, copy, and the
AdamW 16:12 read/write mix), and the rate at which a CU copies global memory
straight into LDS the way the bf16 GEMMs stage their operands.  Each probe is launched on torch's current
stream and timed with events on it; the best of `reps` launches is kept.

Measurement only: nothing here is on the optimizer's path.
"""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libma_peaks.so")
CUS = 256                         # compute units of an MI355X
_lib = None


def load(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libma_peaks.so is not built (%s); run "
                           "`python -m muon_newton_schulz_02_amd.build` first" % path)
    lib = C.CDLL(path)
    lib.ma_peaks_mfma.argtypes = [C.c_int, C.c_int64, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.ma_peaks_lds.argtypes = [C.c_int, C.c_int64, C.c_int, C.c_void_p, C.c_void_p,
                                 C.c_void_p]
    lib.ma_peaks_stream.argtypes = [C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_int64, C.c_void_p, C.c_void_p]
    lib.ma_peaks_dma.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int, C.c_void_p,
                                 C.c_void_p]
    for f in (lib.ma_peaks_mfma, lib.ma_peaks_lds, lib.ma_peaks_stream, lib.ma_peaks_dma):
        f.restype = C.c_int
    _lib = lib
    return lib


def _timed(torch, launch, reps: int) -> float:
    """Best time in ms of `reps` launches (after one untimed launch)."""
    launch()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    return best


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError("%s: hip error %d" % (what, rc))


def mfma(torch, fp32: bool = False, blocks: int = CUS, iters: int = 0, reps: int = 3) -> dict:
    """Dense MFMA rate (TFLOP/s) of independent 32x32 matrix instructions on
    every SIMD, and the shader clock (MHz) during the loop."""
    lib = load()
    iters = iters or (20000 if fp32 else 40000)
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def go():
        _check(lib.ma_peaks_mfma(1 if fp32 else 0, blocks, iters, sink.data_ptr(),
                                 clocks.data_ptr(), st), "ma_peaks_mfma")

    ms = _timed(torch, go, reps)
    flops = blocks * 4.0 * iters * 8 * (4096.0 if fp32 else 32768.0)
    cyc = clocks.view(-1, 2).double()
    mhz = float((cyc[:, 0] / (cyc[:, 1] / 100.0)).median())      # s_memrealtime: 100 MHz
    return {"tflops": flops / (ms * 1e-3) / 1e12, "sclk_mhz": mhz}


def lds(torch, transposing: bool = False, blocks: int = 2 * CUS, iters: int = 4000,
        reps: int = 3) -> dict:
    """LDS read bandwidth: total GB/s, the shader clock during the loop and
    bytes per shader cycle per CU (two 64 KB workgroups per CU, four waves
    each)."""
    lib = load()
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def go():
        _check(lib.ma_peaks_lds(1 if transposing else 0, blocks, iters, sink.data_ptr(),
                                clocks.data_ptr(), st), "ma_peaks_lds")

    ms = _timed(torch, go, reps)
    nbytes = blocks * 4.0 * iters * 16 * (512.0 if transposing else 1024.0)
    cyc = clocks.view(-1, 2).double()
    mhz = float((cyc[:, 0] / (cyc[:, 1] / 100.0)).median())
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"gbps": gbps, "sclk_mhz": mhz, "bytes_per_clk_per_cu": gbps * 1e9 / (mhz * 1e6) / CUS}


def stream(torch, kind: str, gib: float = 1.0, reps: int = 3) -> dict:
    """HBM bytes moved per second by a stream kernel over float4 arrays of
    `gib` GiB each: 'read' (one array read), 'copy' (read one, write
    another), 'adamw_mix' (four arrays read, three written back in place)."""
    lib = load()
    k = {"read": 0, "copy": 1, "adamw_mix": 2}[kind]
    n_vec = int(gib * (1 << 30)) // 16
    n_arr = {0: 1, 1: 2, 2: 4}[k]
    arrs = [torch.ones(n_vec * 4, dtype=torch.float32, device="cuda") * 1e-3 for _ in range(n_arr)]
    while len(arrs) < 4:
        arrs.append(None)
    groups = -(-n_vec // 4096)
    sink = torch.empty(groups * 256 if k == 0 else 1, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    ptr = [a.data_ptr() if a is not None else None for a in arrs]

    def go():
        _check(lib.ma_peaks_stream(k, ptr[0], ptr[1], ptr[2], ptr[3], n_vec, sink.data_ptr(), st),
               "ma_peaks_stream")

    ms = _timed(torch, go, reps)
    per_vec = {0: 16.0, 1: 32.0, 2: 112.0}[k]
    del arrs
    return {"gbps": per_vec * n_vec / (ms * 1e-3) / 1e9}


def dma(torch, src_mib: int, blocks: int = CUS, stages: int = 2048, reps: int = 3) -> dict:
    """Global memory into LDS as the bf16 GEMMs stage operands (one
    workgroup per CU, 32 KB stages, a wait and a barrier per stage), from a
    source of `src_mib` MiB: a few MiB stay in L2, a large source streams
    from the memory-side cache or HBM.  GB/s, shader clock, bytes per shader
    cycle per CU."""
    lib = load()
    nbytes_src = src_mib << 20
    src = torch.ones(nbytes_src // 4, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def go():
        _check(lib.ma_peaks_dma(src.data_ptr(), nbytes_src, blocks, stages, clocks.data_ptr(), st),
               "ma_peaks_dma")

    ms = _timed(torch, go, reps)
    nbytes = blocks * float(stages) * 32768.0
    cyc = clocks.view(-1, 2).double()
    mhz = float((cyc[:, 0] / (cyc[:, 1] / 100.0)).median())
    gbps = nbytes / (ms * 1e-3) / 1e9
    del src
    return {"gbps": gbps, "sclk_mhz": mhz, "bytes_per_clk_per_cu": gbps * 1e9 / (mhz * 1e6) / CUS}


def measure_all(torch) -> dict:
    """Every probe, with the derived per-CU LDS figure."""
    bf = mfma(torch, False)
    f32 = mfma(torch, True)
    l16 = lds(torch, False)
    ltr = lds(torch, True)
    out = {
        "mfma_bf16_tflops": bf["tflops"], "mfma_bf16_sclk_mhz": bf["sclk_mhz"],
        "mfma_fp32_tflops": f32["tflops"], "mfma_fp32_sclk_mhz": f32["sclk_mhz"],
        "lds_read_b128_gbps": l16["gbps"],
        "lds_read_b128_bytes_per_clk_per_cu": l16["bytes_per_clk_per_cu"],
        "lds_read_tr_b64_gbps": ltr["gbps"],
        "lds_read_tr_b64_bytes_per_clk_per_cu": ltr["bytes_per_clk_per_cu"],
        "lds_sclk_mhz": l16["sclk_mhz"],
        "hbm_read_gbps": stream(torch, "read", 4.0)["gbps"],
        "hbm_copy_gbps": stream(torch, "copy", 2.0)["gbps"],
        "hbm_adamw_mix_gbps": stream(torch, "adamw_mix", 1.0)["gbps"],
    }
    near, far = dma(torch, 4), dma(torch, 1024)
    out.update({
        "lds_dma_l2_gbps": near["gbps"],
        "lds_dma_l2_bytes_per_clk_per_cu": near["bytes_per_clk_per_cu"],
        "lds_dma_far_gbps": far["gbps"],
        "lds_dma_far_bytes_per_clk_per_cu": far["bytes_per_clk_per_cu"],
        "lds_dma_sclk_mhz": far["sclk_mhz"],
    })
    torch.cuda.empty_cache()
    return out
