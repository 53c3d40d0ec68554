"""absa_select_noalloc (the selection entry point for callers that cannot allocate) against
absa_select with a caller workspace: the same kernels, so lists and probabilities must be
bit-identical.  Successive calls on one device, each with a smaller problem than the one before,
so later calls run on a scratch buffer that still holds an earlier call's intermediates; then a
problem whose workspace exceeds the fixed 64 MiB is rejected before any launch."""
import ctypes
import sys

import numpy as np
import pytest

from workloads import gen_config, gen_fourier_heads, bf16_round, Workload
from gpu_helpers import dev, problem

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


def _workload(H, T, Hs, Ws, d, Bq, Bk, seed):
    q, k, v = gen_fourier_heads(T, Hs, Ws, d, 8, 0.3, False, seed, list(range(H)))
    L = T * Hs * Ws
    sh = (1, H, L, d)
    return Workload(q=bf16_round(q.reshape(sh)), k=bf16_round(k.reshape(sh)), v=bf16_round(v.reshape(sh)),
                    B=1, H=H, L=L, d=d, T=T, Hs=Hs, Ws=Ws, q_block=Bq, kv_block=Bk, keep=0.2)


def _noalloc_raw(absa, p, q, k, keep, lists, pi, seed, mode):
    """absa_select_noalloc through the C ABI directly (ctypes), on torch's current stream."""
    import torch
    from block_sparse_attention_34_amd import _lib
    lib = absa.library()
    pc = p.c()
    sp = _lib.AbsaSelectParams(float(keep), 4, 3, 0.0, seed, 0, mode)
    bl = lists.c()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.absa_select_noalloc(ctypes.byref(pc), ctypes.byref(sp), q.data_ptr(), k.data_ptr(), ctypes.byref(bl),
                                   pi.data_ptr(), stream)


def _compare_with_workspace_call(absa, wl, keep, seed, mode, tag):
    import torch
    p = problem(wl)
    q, k = dev(wl.q), dev(wl.k)
    ref_lists, ref_pi, _ = absa.select(p, q, k, keep, seed=seed, mode=mode, want_pi=True)
    lists = absa.alloc_lists(p)
    for t in lists:
        t.fill_(-7)                       # stale contents the call must overwrite
    pi = torch.full((p.rows, p.nk), -1.0, dtype=torch.float32, device="cuda")
    st = _noalloc_raw(absa, p, q, k, keep, lists, pi, seed, mode)
    assert st == 0, absa._lib.status_string(st)
    torch.cuda.synchronize()
    count = lists.count.cpu().numpy()
    rc = ref_lists.count.cpu().numpy()
    np.testing.assert_array_equal(count, rc, err_msg=tag)
    kv, rkv = lists.kv_idx.cpu().numpy(), ref_lists.kv_idx.cpu().numpy()
    w, rw = lists.inv_pi.cpu().numpy(), ref_lists.inv_pi.cpu().numpy()
    for r in range(p.rows):
        np.testing.assert_array_equal(kv[r, :count[r]], rkv[r, :count[r]], err_msg=f"{tag} row {r}")
        np.testing.assert_array_equal(w[r, :count[r]].view(np.uint32), rw[r, :count[r]].view(np.uint32),
                                      err_msg=f"{tag} row {r}")
    np.testing.assert_array_equal(pi.cpu().numpy().view(np.uint32), ref_pi.cpu().numpy().view(np.uint32),
                                  err_msg=tag)
    _say(f"{tag}: rows={p.rows} NK={p.nk} mean kept {count.mean():.1f}: bit-identical")


_WL = {}


def _wan14b_one_head():
    # the Wan2.1-14B 720p shape with one head: 60.5 MiB of selection workspace, near the 64 MiB limit
    if "wl" not in _WL:
        _WL["wl"] = gen_config(3, heads=[0])
    return _WL["wl"]


@pytest.mark.parametrize("mode", [0, 1])
def test_noalloc_equals_workspace_call_successive_calls(absa, mode):
    # successive calls, each smaller than the one before: the 720p shape with one head (near the
    # buffer's limit), L = 1200 with ragged tails (d = 128, Bq = 128), the tiny workload (d = 64)
    wl = _wan14b_one_head()
    _compare_with_workspace_call(absa, wl, 0.095, 0, mode, f"mode {mode} call 1 (720p, H=1)")
    mid = _workload(3, 5, 15, 16, 128, 128, 16, seed=61)
    _compare_with_workspace_call(absa, mid, 0.15, 3, mode, f"mode {mode} call 2 (L=1200, H=3, d=128)")
    small = gen_config(1)
    _compare_with_workspace_call(absa, small, 0.25, 0, mode, f"mode {mode} call 3 (L=1024, H=2, d=64)")


def test_noalloc_binding_and_size_limit(absa):
    import torch
    wl = gen_config(1)
    p = problem(wl)
    q, k = dev(wl.q), dev(wl.k)
    lists = absa.alloc_lists(p)
    ref, _, _ = absa.select(p, q, k, 0.25, seed=4)
    absa.select_noalloc(p, q, k, 0.25, lists, seed=4)
    torch.cuda.synchronize()
    assert torch.equal(lists.count, ref.count)
    # 720p Wan shape with one head: about 61 MB of selection workspace fits; 4 heads do not
    big = absa.Problem(1, 5, 75600, 128, 21, 45, 80, 128, 16)
    need = absa.select_workspace_bytes(big, 0.095)
    assert need > 64 << 20
    bl = absa._lib.AbsaBlockList(8, 8, 8, big.nk)   # never dereferenced: rejected before any launch
    pc = big.c()
    sp = absa._lib.AbsaSelectParams(0.095, 0, 0, 0.0, 0, 0, 0)
    st = absa.library().absa_select_noalloc(ctypes.byref(pc), ctypes.byref(sp), 16, 16, ctypes.byref(bl), None,
                                            None)
    assert st == absa._lib.ABSA_ERR_TOO_LARGE
