"""GPU parity of absa_attend_pairs (64-query blocks paired into 128-query rows of the two-row kernel,
over the union of their lists) against the fp64 oracle fed the GPU's own lists: max-abs <= 1e-2,
rel-L2 <= 5e-3, on every row of ragged shapes (an odd number of query blocks, so a head's last pair
holds one block; KV tails inside a tile and, at Bk = 128, in either tile of a block), for SIP, top-k
and all-block lists; empty lists and entries past NK; bf16 output; sampled rows of the Wan2.1-1.3B
480p workload; two runs give the same bytes; and a captured selection + paired attention replays to
the eager result."""
import sys

import numpy as np
import pytest

import oracle as O
from gpu_helpers import (assert_close, dev, errors, gpu_rows, lists_to_host, oracle_rows_from_gpu_lists, problem,
                         sample_rows)
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
                    B=1, H=H, L=L, d=d, T=T, Hs=Hs, Ws=Ws, q_block=64, kv_block=Bk, keep=0.3)


def _check(absa, wl, p, lists, rows, tag):
    import torch
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    o2 = absa.attend_pairs(p, q, k, v, lists)
    o1 = absa.attend(p, q, k, v, lists)
    torch.cuda.synchronize()
    o2, o1 = o2.cpu().numpy(), o1.cpu().numpy()
    count, kv, w = lists_to_host(lists)
    ref = oracle_rows_from_gpu_lists(wl, 64, wl.kv_block, count, kv, w, rows, p.sigma)
    g2, g1 = gpu_rows(o2, wl, 64, rows), gpu_rows(o1, wl, 64, rows)
    got = np.concatenate([g2[r] for r in rows])
    err = assert_close(got, np.concatenate([ref[r] for r in rows]), tag)
    d1 = errors(got, np.concatenate([g1[r] for r in rows]))
    _say(f"{tag}: rows={len(rows)} vs oracle max_abs={err[0]:.3e} rel_l2={err[1]:.3e}; "
         f"vs the one-row kernel max_abs={d1[0]:.3e}")
    assert d1[0] <= 1e-2
    return o2


@pytest.mark.parametrize("d,Bk,grid", [(128, 16, (5, 15, 16)), (64, 16, (5, 15, 16)), (128, 32, (3, 7, 9)),
                                       (128, 64, (5, 15, 13)), (128, 128, (5, 15, 13)), (64, 128, (5, 15, 16))])
def test_pairs_match_oracle(absa, d, Bk, grid):
    # L = 1200 (19 query blocks), 189 (3) and 975 (16, ragged KV tail)
    wl = _workload(2, *grid, d, Bk, seed=31 + d + Bk)
    p = problem(wl)
    rows = list(range(p.rows))
    for mode in (O.SEL_SIP, O.SEL_TOPK, O.SEL_ALL):
        lists, _, _ = absa.select(p, dev(wl.q), dev(wl.k), 0.3, seed=4, mode=mode)
        _check(absa, wl, p, lists, rows, f"pairs d={d} Bk={Bk} L={wl.L} mode {mode}")


def test_pairs_empty_lists_and_invalid_entries(absa):
    import torch
    wl = _workload(1, 1, 12, 16, 128, 16, seed=9)  # L = 192: query blocks 0, 1 pair up, block 2 alone
    p = problem(wl)
    assert p.nq == 3 and p.nk == 12
    count = torch.tensor([0, 3, 2], dtype=torch.int32).cuda()
    kv = torch.tensor([[0] * 4, [2, 7, 99, 0], [1, 7, 0, 0]], dtype=torch.int32).cuda()  # 99 >= NK: skipped
    w = torch.tensor([[1.0] * 4, [2.0, 1.5, 1.0, 1.0], [3.0, 1.25, 1.0, 1.0]], dtype=torch.float32).cuda()
    lists = absa.BlockLists(count, kv, w)
    o = absa.attend_pairs(p, dev(wl.q), dev(wl.k), dev(wl.v), lists).cpu().numpy()
    assert (o[0, 0, :64] == 0).all()
    ref1 = O.attend_row_block(wl.q, wl.k, wl.v, 0, 1, 64, 16, [2, 7], [2.0, 1.5], p.sigma)
    ref2 = O.attend_row_block(wl.q, wl.k, wl.v, 0, 2, 64, 16, [1, 7], [3.0, 1.25], p.sigma)
    assert_close(o[0, 0, 64:128], ref1, "pair member with an invalid entry")
    assert_close(o[0, 0, 128:], ref2, "unpaired last block")


def test_pairs_bf16_output_and_repeatability(absa):
    import torch
    wl = _workload(2, 3, 7, 9, 128, 16, seed=12)
    p = problem(wl, out_bf16=True)
    lists, _, _ = absa.select(p, dev(wl.q), dev(wl.k), 0.3, seed=1)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    o = absa.attend_pairs(p, q, k, v, lists)
    o2 = absa.attend_pairs(p, q, k, v, lists)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    count, kv, w = lists_to_host(lists)
    rows = list(range(p.rows))
    ref = oracle_rows_from_gpu_lists(wl, 64, 16, count, kv, w, rows, p.sigma)
    got = gpu_rows(o.float().cpu().numpy(), wl, 64, rows)
    g, rr = np.concatenate([got[r] for r in rows]), np.concatenate([ref[r] for r in rows])
    # bf16 output adds half an ulp of |o| (<= 2^-9 relative)
    assert (np.abs(g - rr) <= 1e-2 + 2.0 ** -8 * np.abs(rr)).all()


def test_pairs_wan13b_480p_sampled_rows(absa):
    wl = gen_config(2)
    p = problem(wl)
    lists, _, _ = absa.select(p, dev(wl.q), dev(wl.k), 0.10, seed=0)
    rows = sample_rows(p.nq, wl.H, 40, seed=77)
    _check(absa, wl, p, lists, rows, "pairs Wan2.1-1.3B 480p (sampled rows)")


def test_pairs_graph_capture_replays_match_eager(absa):
    # absa_attend_pairs allocates nothing (its union lists live in the caller's workspace) and
    # sets no memory, so selection + paired attention can be captured; every replay, with eager
    # work clobbering the outputs and the workspace in between, reproduces the eager result
    import torch
    wl = _workload(2, 5, 15, 16, 128, 16, seed=13)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists = absa.alloc_lists(p)
    ws = torch.empty(absa.select_workspace_bytes(p, 0.2), dtype=torch.uint8, device="cuda")
    pws = torch.empty(absa.attend_pairs_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    o = torch.empty((p.B, p.H, p.L, p.d), dtype=torch.float32, device="cuda")

    def step():
        absa.select(p, q, k, 0.2, seed=5, lists=lists, workspace=ws)
        absa.attend_pairs(p, q, k, v, lists, out=o, workspace=pws)

    def clobber():
        o.zero_()
        lists.count.zero_()
        lists.kv_idx.zero_()
        lists.inv_pi.zero_()
        pws.fill_(0xFF)

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
