"""Binding of libwa_diag.so (include/wa_diag.h): the matrix-core ceiling
probe that sets the attention kernels' rates against what the GPU sustains
when they are measured.  Not part of the attention path."""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
DIAG_LIB_PATH = os.path.join(_PKG, "libwa_diag.so")

FLOP_PER_MFMA = {"bf16": 32 * 32 * 16 * 2, "fp8": 32 * 32 * 64 * 2}
_DTYPE = {"bf16": 0, "fp8": 1}


def _load():
    if not os.path.exists(DIAG_LIB_PATH):
        raise ImportError(f"{DIAG_LIB_PATH} is missing: run python whisper_attention_amd/build.py")
    lib = ctypes.CDLL(DIAG_LIB_PATH)
    lib.wa_diag_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.wa_diag_mfma_ceiling.restype = ctypes.c_int
    lib.wa_diag_sclk_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.wa_diag_sclk_probe.restype = ctypes.c_int
    lib.wa_diag_wall_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int)]
    lib.wa_diag_wall_clock_khz.restype = ctypes.c_int
    return lib


lib = _load()
EXPORTED = ("wa_diag_mfma_ceiling", "wa_diag_sclk_probe", "wa_diag_wall_clock_khz")


def mfma_ceiling(dtype="bf16", blocks_per_cu=2, iters=4096, reps=10):
    """Run the probe ``reps`` times on the current device and stream; returns
    the sustained rate (TFLOP/s, from events around the repetitions) and the
    shader clock the first wave of each block saw (MHz, mean over blocks)."""
    dev = torch.cuda.current_device()
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    n_blocks = blocks_per_cu * n_cu
    ticks = torch.zeros((n_blocks, 2), dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    khz = ctypes.c_int(0)
    if lib.wa_diag_wall_clock_khz(ctypes.byref(khz)) != 0:
        raise RuntimeError("wa_diag_wall_clock_khz failed")

    def call():
        st = lib.wa_diag_mfma_ceiling(_DTYPE[dtype], n_blocks, iters, ticks.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"wa_diag_mfma_ceiling returned {st}")

    for _ in range(3):
        call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        call()
    ev[1].record()
    torch.cuda.synchronize()
    sec = ev[0].elapsed_time(ev[1]) * 1e-3 / reps
    flop = float(n_blocks) * 4 * iters * 4 * FLOP_PER_MFMA[dtype]
    t = ticks.cpu().numpy().astype("float64")
    ok = t[:, 1] > 0
    mhz = float((t[ok, 0] / t[ok, 1]).mean() * khz.value / 1e3) if ok.any() else None
    return {"TFLOP/s": round(flop / sec / 1e12, 1), "sclk_MHz": None if mhz is None else round(mhz, 0),
            "us_per_call": round(sec * 1e6, 1), "blocks": n_blocks, "iters": iters,
            "wall_clock_kHz": khz.value}


class SclkProbe:
    """The shader clock right after the work enqueued before it: ``launch()``
    enqueues the probe on the current stream (no synchronization), ``mhz()``
    synchronizes and returns the mean over its blocks of the measured
    launches since the last read."""

    def __init__(self, n_blocks=8, spin=500):
        self.n_blocks, self.spin = n_blocks, spin
        self.khz = ctypes.c_int(0)
        if lib.wa_diag_wall_clock_khz(ctypes.byref(self.khz)) != 0:
            raise RuntimeError("wa_diag_wall_clock_khz failed")
        self.bufs, self.used = [], 0

    def launch(self):
        if self.used == len(self.bufs):
            self.bufs.append(torch.zeros((self.n_blocks, 2), dtype=torch.int64, device="cuda"))
        t = self.bufs[self.used]
        self.used += 1
        st = lib.wa_diag_sclk_probe(self.n_blocks, self.spin, t.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"wa_diag_sclk_probe returned {st}")

    def mhz(self):
        torch.cuda.synchronize()
        vals = []
        for t in self.bufs[:self.used]:
            a = t.cpu().numpy().astype("float64")
            ok = a[:, 1] > 0
            vals.extend(list(a[ok, 0] / a[ok, 1] * self.khz.value / 1e3))
        self.used = 0
        return None if not vals else round(float(sum(vals) / len(vals)), 0)
