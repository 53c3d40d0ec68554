"""Per-clock issue rates of the units the gather-attention kernel leans on (tests/hip/unit_rates_probe.hip,
built by __graft_entry__.build()): LDS reads (16-byte and transposing 8-byte), v_exp_f32, v_fma_f32 and
v_mfma_f32_32x32x16_bf16, alone (one or two waves per SIMD) and with a matrix wave and a vector wave
sharing each SIMD.  The figures are printed (run with -s) and feed the kernel's bound analysis; the
assertions only check that every wave measured its own loop and that the rates are physically sensible."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libunit_rates_probe.so")
NBLK = 256          # one workgroup per CU (96 KB of LDS each)
ITERS = 4000

# per-iteration work of a wave in each mode: (instructions, LDS bytes)
MODES = {1: ("ds_read_b128", 8, 8 * 64 * 16), 2: ("ds_read_b64_tr_b16", 8, 8 * 64 * 8),
         3: ("v_exp_f32", 16, 0), 4: ("v_fma_f32", 16, 0), 5: ("v_mfma_f32_32x32x16_bf16", 4, 0)}


def _run(lib, modes):
    """Per-workgroup counters of one launch: arrays [NBLK, 8] of loop start / end clock counts and
    real-time (100 MHz) counts."""
    import torch
    md = torch.tensor(modes, dtype=torch.int32, device="cuda")
    cyc = torch.zeros(NBLK * 32, dtype=torch.int64, device="cuda")
    sink = torch.empty(NBLK * 512, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(2):  # the first launch warms the clock up
        assert lib.unit_rates_probe(md.data_ptr(), ITERS, cyc.data_ptr(), sink.data_ptr(), NBLK, st) == 0
    torch.cuda.synchronize()
    c = cyc.cpu().numpy().reshape(NBLK, 8, 4).astype(np.float64)
    return c[..., 0], c[..., 1], c[..., 2], c[..., 3]


def _span(t0, t1, waves):
    """Median over the workgroups of the clock span from the first start to the last end of ``waves``."""
    w = list(waves)
    return float(np.median(t1[:, w].max(axis=1) - t0[:, w].min(axis=1)))


def _clock_ghz(t0, t1, r0, r1, waves):
    w = list(waves)
    cyc = t1[:, w].max(axis=1) - t0[:, w].min(axis=1)
    ns = (r1[:, w].max(axis=1) - r0[:, w].min(axis=1)) * 10.0
    return float(np.median(cyc / ns))


def _say(msg):
    print(msg, flush=True)


def test_unit_rates():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB)
    lib.unit_rates_probe.restype = ctypes.c_int
    lib.unit_rates_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p]
    rows = []
    for m, (name, n_inst, lds_b) in MODES.items():
        for wps in (1, 2):  # waves per SIMD running the mode (waves w and w + 4 share SIMD w)
            modes = [m] * 4 + [m if wps == 2 else 0] * 4
            t0, t1, r0, r1 = _run(lib, modes)
            act = range(4 * wps)
            assert np.all(t1[:, act] > t0[:, act])
            span = _span(t0, t1, act)
            per_inst = span / (ITERS * n_inst * wps)  # cycles per instruction per SIMD
            lds = lds_b * 4 * wps * ITERS / span if lds_b else None
            ghz = _clock_ghz(t0, t1, r0, r1, act)
            rows.append((name, wps, per_inst, lds))
            _say(f"{name:26s} waves/SIMD {wps}: {per_inst:6.2f} cycles per instruction per SIMD"
                 + (f", LDS {lds:6.1f} B/clk/CU" if lds else "") + f" (clock {ghz:.2f} GHz)")
    # a matrix wave and a vector (or LDS) wave on every SIMD
    mf = [r for r in rows if r[0].startswith("v_mfma") and r[1] == 1][0]
    for m in (3, 4, 1, 2):
        name, n_inst, lds_b = MODES[m]
        t0, t1, r0, r1 = _run(lib, [5] * 4 + [m] * 4)
        mm = _span(t0, t1, range(4)) / (ITERS * 4)
        vv = _span(t0, t1, range(4, 8)) / (ITERS * n_inst)
        both = _span(t0, t1, range(8)) / ITERS
        solo = [r for r in rows if r[0] == name and r[1] == 1][0]
        alone_sum = mf[2] * 4 + solo[2] * n_inst
        _say(f"mfma wave + {name:20s} wave per SIMD: mfma {mm:6.2f} cycles/inst (alone {mf[2]:.2f}), {name} "
             f"{vv:6.2f} cycles/inst (alone {solo[2]:.2f}); both loops {both:7.1f} cycles per iteration against "
             f"{alone_sum:7.1f} one after the other")
        assert mm > 0 and vv > 0
    # sanity: the specification's 2.5 PFLOP/s at 2.4 GHz is one 32x32x16 product per 32 cycles and SIMD
    assert 16.0 <= mf[2] <= 256.0
