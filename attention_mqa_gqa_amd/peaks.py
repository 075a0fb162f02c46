"""Binding of libmqa_peaks.so (include/mqa_peaks.h): measured ceilings of the
device -- the bf16 MFMA rate and the clock it runs at, HBM read and copy
bandwidth, LDS read bandwidth -- against which the attention kernels'
roofline fractions are also reported.  Argument marshalling and timing only.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmqa_peaks.so")

EXPORTED_SYMBOLS = (
    "mqa_peak_compute_units",
    "mqa_peak_sink_floats",
    "mqa_peak_mfma_bf16",
    "mqa_peak_hbm_read",
    "mqa_peak_hbm_copy",
    "mqa_peak_lds_read",
)

MFMA, READ, LDS = 0, 1, 2


def load():
    import torch  # noqa: F401  (bind to torch's HIP runtime, as the attention library does)
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python attention_mqa_gqa_amd/build.py`")
    l = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    l.mqa_peak_compute_units.restype = i
    l.mqa_peak_compute_units.argtypes = []
    l.mqa_peak_sink_floats.restype = sz
    l.mqa_peak_sink_floats.argtypes = [i, i]
    l.mqa_peak_mfma_bf16.restype = i
    l.mqa_peak_mfma_bf16.argtypes = [i, i, vp, vp, vp]
    l.mqa_peak_hbm_read.restype = i
    l.mqa_peak_hbm_read.argtypes = [vp, sz, vp, vp]
    l.mqa_peak_hbm_copy.restype = i
    l.mqa_peak_hbm_copy.argtypes = [vp, vp, sz, vp]
    l.mqa_peak_lds_read.restype = i
    l.mqa_peak_lds_read.argtypes = [i, i, vp, vp]
    return l


def _time(torch, launch, reps):
    """Mean milliseconds of `launch()` over `reps` launches after two warm-ups."""
    stream = torch.cuda.current_stream()
    for _ in range(2):
        launch(stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        launch(stream.cuda_stream)
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def measure(read_mib=4096):
    """Run every probe on cuda:0; returns a dict of measured ceilings."""
    import torch
    l = load()
    dev = torch.device("cuda:0")
    ncu = l.mqa_peak_compute_units()

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: status {st}")

    res = {"compute_units": ncu}
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    for wps in (1, 2):
        sink = torch.empty(l.mqa_peak_sink_floats(MFMA, wps), dtype=torch.float32, device=dev)
        iters = 4000
        ms = _time(torch, lambda s: check(l.mqa_peak_mfma_bf16(wps, iters, sink.data_ptr(), clocks.data_ptr(), s),
                                          "mfma"), 10)
        flop = ncu * 4 * wps * iters * 8 * 32768
        c = clocks.cpu().tolist()
        res[f"mfma_bf16_tflops_{wps}wave"] = round(flop / (ms * 1e-3) / 1e12, 1)
        res[f"mfma_clock_ghz_{wps}wave"] = round(c[0] / (c[1] / 100e6) / 1e9, 3) if c[1] > 0 else None
    n = read_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(3)
    sink = torch.empty(l.mqa_peak_sink_floats(READ, 1), dtype=torch.float32, device=dev)
    ms = _time(torch, lambda s: check(l.mqa_peak_hbm_read(src.data_ptr(), n, sink.data_ptr(), s), "read"), 10)
    res["hbm_read_gbs"] = round(n / (ms * 1e-3) / 1e9, 1)
    half = n // 2
    ms = _time(torch, lambda s: check(l.mqa_peak_hbm_copy(src.data_ptr(), src.data_ptr() + half, half, s),
                                      "copy"), 10)
    res["hbm_copy_gbs"] = round(2 * half / (ms * 1e-3) / 1e9, 1)
    del src
    for w in (4, 8):
        sink = torch.empty(l.mqa_peak_sink_floats(LDS, w), dtype=torch.float32, device=dev)
        iters = 20000
        ms = _time(torch, lambda s: check(l.mqa_peak_lds_read(w, iters, sink.data_ptr(), s), "lds"), 5)
        res[f"lds_read_tbs_{w}wave"] = round(ncu * w * iters * 8 * 1024 / (ms * 1e-3) / 1e12, 2)
    return res
