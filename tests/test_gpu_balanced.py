"""GPU checks of absa_attend_balanced (the persistent grid with per-XCD work queues): its output is
bit-identical to absa_attend's on ragged 128-query shapes (d 64 and 128, KV blocks of 16 to 128 keys),
with SIP lists, empty lists and entries past NK, bf16 output, more row pairs than workgroups (a
partial last run of 256 pairs included) and fewer; it matches the fp64 oracle fed the same lists;
repeated calls on one workspace, and a smaller problem after a larger one, give the same bytes; a
captured selection + balanced attention replays to the eager result; and at the Wan2.1-14B-shaped
720p workload it reproduces absa_attend bit for bit."""
import sys

import numpy as np
import pytest

from gpu_helpers import assert_close, dev, gpu_rows, lists_to_host, oracle_rows_from_gpu_lists, problem
from workloads import Workload, bf16_round, gen_config, gen_fourier_heads

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


def _workload(H, T, Hs, Ws, d, Bk, seed):
    q, k, v = gen_fourier_heads(T, Hs, Ws, d, 8, 0.3, False, seed, list(range(H)))
    L = T * Hs * Ws
    sh = (1, H, L, d)
    return Workload(q=bf16_round(q.reshape(sh)), k=bf16_round(k.reshape(sh)), v=bf16_round(v.reshape(sh)),
                    B=1, H=H, L=L, d=d, T=T, Hs=Hs, Ws=Ws, q_block=128, kv_block=Bk, keep=0.2)


def _both(absa, p, q, k, v, lists, ws=None):
    import torch
    o1 = absa.attend(p, q, k, v, lists)
    o2 = absa.attend_balanced(p, q, k, v, lists, workspace=ws)
    torch.cuda.synchronize()
    return o1, o2


@pytest.mark.parametrize("d,Bk,H,grid", [(128, 16, 2, (5, 15, 16)), (64, 16, 3, (5, 15, 13)),
                                         (128, 32, 2, (3, 7, 9)), (128, 64, 2, (5, 15, 13)),
                                         (128, 128, 2, (5, 15, 13)), (64, 128, 1, (4, 16, 16))])
def test_balanced_is_bit_identical_to_attend(absa, d, Bk, H, grid):
    import torch
    wl = _workload(H, *grid, d, Bk, seed=21 + d + Bk)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists, _, _ = absa.select(p, q, k, 0.2, seed=3)
    o1, o2 = _both(absa, p, q, k, v, lists)
    assert torch.equal(o1, o2)
    _say(f"d={d} Bk={Bk} L={wl.L} rows={p.rows}: bit-identical")


def test_balanced_matches_oracle(absa):
    wl = _workload(2, 5, 15, 16, 128, 16, seed=7)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists, _, _ = absa.select(p, q, k, 0.2, seed=9)
    o = absa.attend_balanced(p, q, k, v, lists).cpu().numpy()
    count, kv, w = lists_to_host(lists)
    rows = list(range(p.rows))
    ref = oracle_rows_from_gpu_lists(wl, 128, 16, count, kv, w, rows, p.sigma)
    got = gpu_rows(o, wl, 128, rows)
    err = assert_close(np.concatenate([got[r] for r in rows]), np.concatenate([ref[r] for r in rows]), "balanced")
    _say(f"all {len(rows)} rows vs oracle: max_abs={err[0]:.3e} rel_l2={err[1]:.3e}")


def test_balanced_more_pairs_than_workgroups(absa):
    # 10 heads x 60 query blocks = 300 row pairs: one full run of 256 pairs and a partial one, more
    # pairs than there are workgroups, so workgroups take several pairs and the last from other queues
    import torch
    wl = _workload(10, 8, 30, 32, 64, 16, seed=31)
    p = problem(wl)
    assert (p.rows + 1) // 2 == 300
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists, _, _ = absa.select(p, q, k, 0.1, seed=4)
    ws = torch.empty(absa.attend_balanced_workspace_bytes(), dtype=torch.uint8, device="cuda")
    o1, o2 = _both(absa, p, q, k, v, lists, ws)
    assert torch.equal(o1, o2)
    o3 = absa.attend_balanced(p, q, k, v, lists, workspace=ws)  # the same workspace again
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)
    # then a smaller problem on the same workspace
    wl2 = _workload(1, 5, 15, 13, 64, 16, seed=32)
    p2 = problem(wl2)
    q2, k2, v2 = dev(wl2.q), dev(wl2.k), dev(wl2.v)
    lists2, _, _ = absa.select(p2, q2, k2, 0.2, seed=4)
    o4, o5 = _both(absa, p2, q2, k2, v2, lists2, ws)
    assert torch.equal(o4, o5)


def test_balanced_empty_lists_invalid_entries_bf16(absa):
    import torch
    wl = _workload(2, 5, 15, 16, 128, 32, seed=41)
    for out_bf16 in (False, True):
        p = problem(wl, out_bf16=out_bf16)
        q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
        lists, _, _ = absa.select(p, q, k, 0.3, seed=6)
        count = lists.count.clone()
        count[1::5] = 0                                   # empty lists: those rows are 0
        lists.count.copy_(count)
        kv = lists.kv_idx.clone()
        kv[2::7, 0] = p.nk + 5                            # an entry past NK is skipped
        lists.kv_idx.copy_(kv)
        o1, o2 = _both(absa, p, q, k, v, lists)
        assert torch.equal(o1, o2), f"out_bf16={out_bf16}"


def test_balanced_graph_capture_replays_match_eager(absa):
    # the queues are cleared by a kernel on the stream, not a memory set, so selection + balanced
    # attention can be captured; every replay, with eager work clobbering the outputs, the lists and
    # the queues in between, reproduces the eager result
    import torch
    wl = _workload(2, 5, 15, 16, 128, 16, seed=51)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists = absa.alloc_lists(p)
    ws = torch.empty(absa.select_workspace_bytes(p, 0.2), dtype=torch.uint8, device="cuda")
    qws = torch.empty(absa.attend_balanced_workspace_bytes(), dtype=torch.uint8, device="cuda")
    o = torch.empty((p.B, p.H, p.L, p.d), dtype=torch.float32, device="cuda")

    def step():
        absa.select(p, q, k, 0.2, seed=5, lists=lists, workspace=ws)
        absa.attend_balanced(p, q, k, v, lists, out=o, workspace=qws)

    def clobber():
        o.zero_()
        lists.count.zero_()
        lists.kv_idx.zero_()
        lists.inv_pi.zero_()
        qws.fill_(0xFF)

    clobber()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (lists.count, lists.kv_idx, lists.inv_pi, o)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        clobber()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((lists.count, lists.kv_idx, lists.inv_pi, o), ref):
            assert torch.equal(a, b), f"replay {i}"


def test_balanced_wan14b_720p_bit_identical(absa):
    import torch
    wl = gen_config(3)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists, _, _ = absa.select(p, q, k, 0.095, seed=0)
    o1, o2 = _both(absa, p, q, k, v, lists)
    assert torch.equal(o1, o2)
    _say(f"720p: {p.rows} rows, bit-identical")
