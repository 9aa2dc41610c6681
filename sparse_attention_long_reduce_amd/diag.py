"""Binding of the measurement helpers (include/cpa_diag.h): argument marshalling only."""
import ctypes

import torch

from ._lib import CpaError, load_diag

MFMA_FLOP = 32 * 32 * 16 * 2   # one v_mfma_f32_32x32x16_bf16


def clock_rates(device=0):
    """(peak engine clock, constant wall-clock rate) of the device in kHz, as HIP reports them."""
    eng, wall = ctypes.c_int(0), ctypes.c_int(0)
    st = load_diag().cpa_diag_clock_rates(int(device), ctypes.byref(eng), ctypes.byref(wall))
    if st != 0:
        raise CpaError(st, "cpa_diag_clock_rates")
    return eng.value, wall.value


def mfma_peak(device=0, iters=20000, threads=512, reps=3):
    """Rate of the bf16 matrix cores on a loop of independent MFMAs, one workgroup per compute
    unit (threads / 256 waves per SIMD), timed with HIP events on the current stream; the best of
    `reps` launches.  Also the engine clock during that launch, from the shader-clock cycles over
    the constant-rate clock ticks of workgroup 0."""
    dev = torch.device("cuda", device) if isinstance(device, int) else device
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(n_cu * threads, dtype=torch.float32, device=dev)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    _, wall_khz = clock_rates(dev.index or 0)
    lib = load_diag()
    flop = n_cu * (threads // 64) * iters * 4 * MFMA_FLOP
    best = None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev)
        for _ in range(reps + 1):   # the first launch warms up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            st = lib.cpa_diag_mfma_loop(n_cu, threads, iters, sink.data_ptr(), clk.data_ptr(), stream.cuda_stream)
            e1.record()
            if st != 0:
                raise CpaError(st, "cpa_diag_mfma_loop")
            torch.cuda.synchronize(dev)
            ms = e0.elapsed_time(e1)
            cycles, ticks = (int(x) for x in clk.cpu().tolist())
            mhz = cycles / (ticks / (wall_khz * 1e3)) / 1e6 if ticks > 0 else 0.0
            r = {"tflops": flop / (ms * 1e-3) / 1e12, "ms": ms, "engine_clock_mhz": mhz}
            if best is None or r["tflops"] > best["tflops"]:
                best = r
    best.update({"flop_per_launch": flop, "workgroups": n_cu, "waves_per_simd": threads // 256,
                 "iters": iters})
    return best
