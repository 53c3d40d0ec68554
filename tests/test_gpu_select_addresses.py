"""Selection with its workspace and probability output at device addresses whose low 32 bits have
bit 31 set.  The kernels build buffer resources from wave-uniform pointers; a low half taken as a
signed 32-bit value would be sign-extended into the high half and turn such an address into an
invalid one.  These calls place both buffers there on purpose and must give the same lists,
weights and probabilities, bit for bit, as a call on torch-allocated memory."""
import ctypes
import sys

import numpy as np
import pytest

import oracle as O
from workloads import gen_exact, gen_config
from gpu_helpers import dev, lists_to_host, problem

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def absa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import block_sparse_attention_34_amd as m
    m.library()
    return m


def _high_half_views(nbytes_a, nbytes_b):
    """Two adjacent byte views (256-aligned) of one allocation whose start addresses have bit 31 of
    their low 32 bits set."""
    import torch
    span = nbytes_a + nbytes_b + 512
    buf = torch.empty(span + (1 << 31), dtype=torch.uint8, device="cuda")
    lo = buf.data_ptr() & 0xFFFFFFFF
    off = 0 if lo >= (1 << 31) else (1 << 31) - lo
    off = (off + 255) & ~255
    a0 = off
    b0 = (a0 + nbytes_a + 255) & ~255
    assert b0 + nbytes_b <= buf.numel()
    for start in (a0, b0):
        assert (buf.data_ptr() + start) & 0x80000000
    return buf, buf[a0:a0 + nbytes_a], buf[b0:b0 + nbytes_b]


@pytest.mark.parametrize("case", ["integer", "tiny"])
@pytest.mark.parametrize("mode", [O.SEL_SIP, O.SEL_TOPK])
def test_select_at_addresses_with_bit31_set(absa, case, mode):
    import torch
    wl = gen_exact(0) if case == "integer" else gen_config(1)
    p = problem(wl)
    q, k = dev(wl.q), dev(wl.k)
    ref_lists, ref_pi, _ = absa.select(p, q, k, 0.25, seed=3, mode=mode, want_pi=True)
    torch.cuda.synchronize()
    nbytes = absa.select_workspace_bytes(p, 0.25, mode=mode)
    buf, ws, pib = _high_half_views(nbytes, p.rows * p.nk * 4)
    _say(f"{case} mode {mode}: workspace at {ws.data_ptr():#x}, pi at {pib.data_ptr():#x}")
    lists = absa.alloc_lists(p)
    pc = p.c()
    sp = absa._params(0.25, 0, 0, 0.0, 3, 0, mode)
    bl = lists.c()
    st = absa.library().absa_select(ctypes.byref(pc), ctypes.byref(sp), q.data_ptr(), k.data_ptr(),
                                    ctypes.byref(bl), ctypes.c_void_p(pib.data_ptr()),
                                    ctypes.c_void_p(ws.data_ptr()), nbytes, absa._stream())
    assert st == 0
    torch.cuda.synchronize()
    c0, k0, w0 = lists_to_host(ref_lists)
    c1, k1, w1 = lists_to_host(lists)
    np.testing.assert_array_equal(c0, c1)
    for r in range(p.rows):
        np.testing.assert_array_equal(k0[r, :c0[r]], k1[r, :c1[r]])
        np.testing.assert_array_equal(w0[r, :c0[r]].view(np.uint32), w1[r, :c1[r]].view(np.uint32))
    pi1 = pib.view(torch.float32).view(p.rows, p.nk).cpu().numpy()
    np.testing.assert_array_equal(ref_pi.cpu().numpy().view(np.uint32), pi1.view(np.uint32))
    del buf
