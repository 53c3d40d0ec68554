"""The selection kernels form 2^(l - m) with v_exp_f32 and rely on it being exact at integer
arguments (so that integer logits give exact terms and the integer workloads' selection is exact):
checked on the device for every integer in [-126, 125] (tests/hip/exp2_probe.hip, built by
__graft_entry__.build()); and, at non-integer arguments, within 2 ulp of the correctly rounded
power."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libexp2_probe.so")


def test_exp2_is_exact_at_integers():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB)
    lib.exp2_probe.restype = ctypes.c_int
    lib.exp2_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    ints = np.arange(-126, 126, dtype=np.float32)
    rng = np.random.default_rng(3)
    frac = rng.uniform(-64.0, 0.0, 4096).astype(np.float32)
    x = np.concatenate([ints, frac])
    xd = torch.from_numpy(x).cuda()
    yd = torch.empty_like(xd)
    assert lib.exp2_probe(xd.data_ptr(), yd.data_ptr(), x.size, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    np.testing.assert_array_equal(y[:ints.size], np.ldexp(np.float32(1.0), ints.astype(np.int32)).astype(np.float32))
    exact = np.exp2(frac.astype(np.float64))
    ulp = np.spacing(exact.astype(np.float32)).astype(np.float64)
    assert (np.abs(y[ints.size:].astype(np.float64) - exact) <= 2.0 * ulp).all()
