"""ctypes binding of libmiclock.so (include/miclock.h): the engine clock the
GPU holds while other work runs, from a probe that reads the shader-clock
cycle counter over a window of the 100 MHz real-time counter.

Measurement tooling beside the attention library (the benchmark reports the
clock its main kernel ran at); it raises when the library is not built.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmiclock.so")
REALTIME_HZ = 100_000_000  # s_memrealtime rate

_lib = None


def library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m exact_io_aware_attn_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.miclock_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                      ctypes.c_uint64, ctypes.c_void_p]
        lib.miclock_probe.restype = ctypes.c_int
        _lib = lib
    return _lib


class ClockProbe:
    """Probe workgroups (one per XCD by default, two rounds of 8) writing into
    a device buffer; start() enqueues them on `stream`, result() reads them."""

    def __init__(self, n_groups=16, device="cuda:0"):
        import torch
        self.n = n_groups
        self.out = torch.zeros((n_groups, 4), dtype=torch.int64, device=device)

    def start(self, window_s, warm_s=0.0, stream=None):
        import torch
        stream = stream if stream is not None else torch.cuda.current_stream()
        with torch.cuda.stream(stream):  # cleared in order with the probe's own writes
            self.out.zero_()
        st = library().miclock_probe(
            ctypes.c_void_p(self.out.data_ptr()), self.n, int(warm_s * REALTIME_HZ),
            max(1, int(window_s * REALTIME_HZ)), ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"miclock_probe failed with status {st}")

    def result(self):
        """Per probe MHz (after the probe's stream has finished), in launch
        order; probe i ran on XCD i mod 8."""
        o = self.out.cpu().tolist()
        return [c / r * (REALTIME_HZ / 1e6) if r > 0 else float("nan") for c, r, _, _ in o]


def summary(mhz):
    """min / mean / max over the XCDs (probes i and i + 8 share one)."""
    per_xcd = []
    for x in range(min(8, len(mhz))):
        v = mhz[x::8]
        per_xcd.append(sum(v) / len(v))
    return {"mhz_min": min(per_xcd), "mhz_mean": sum(per_xcd) / len(per_xcd),
            "mhz_max": max(per_xcd), "mhz_per_xcd": per_xcd}
