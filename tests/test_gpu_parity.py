"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on seeded inputs.

Attention outputs are compared with the oracle fed the GPU's own block lists (max-abs <= 1e-2,
rel-L2 <= 5e-3).  Selection is bit-exact on the integer workload and agrees on >= 99.9% of
block decisions on the Fourier workloads."""
import math
import sys

import numpy as np
import pytest

import oracle as O
from workloads import gen_config, gen_exact, gen_fourier_heads, bf16_round, Workload
from gpu_helpers import (AGREE, assert_close, decision_agreement, dev, errors, gpu_rows, keep32,
                         lists_to_host, oracle_rows_from_gpu_lists, problem, sample_rows)

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


def _random_workload(H, T, Hs, Ws, d, Bq, Bk, seed, keep=0.25, modes=4):
    q, k, v = gen_fourier_heads(T, Hs, Ws, d, modes, 0.3, False, seed, list(range(H)))
    L = T * Hs * Ws
    sh = (1, H, L, d)
    return Workload(q=bf16_round(q.reshape(sh)), k=bf16_round(k.reshape(sh)), v=bf16_round(v.reshape(sh)),
                    B=1, H=H, L=L, d=d, T=T, Hs=Hs, Ws=Ws, q_block=Bq, kv_block=Bk, keep=keep)


# ----------------------------------------------------------------------------- dense (pi = 1)

@pytest.mark.parametrize("shape", [
    dict(H=2, T=4, Hs=16, Ws=16, d=64, Bq=64),      # the tiny workload's shape
    dict(H=2, T=3, Hs=7, Ws=9, d=128, Bq=128),      # L = 189: ragged query and key tails
    dict(H=3, T=5, Hs=9, Ws=13, d=64, Bq=128),      # L = 585
    dict(H=1, T=1, Hs=1, Ws=1, d=128, Bq=64),       # L = 1
])
def test_dense_matches_oracle(absa, shape):
    wl = _random_workload(shape["H"], shape["T"], shape["Hs"], shape["Ws"], shape["d"], shape["Bq"], 16,
                          seed=11)
    p = problem(wl)
    o = absa.dense(p, dev(wl.q), dev(wl.k), dev(wl.v)).cpu().numpy()
    ref = np.stack([O.dense_attention(wl.q[0, h], wl.k[0, h], wl.v[0, h], p.sigma) for h in range(wl.H)])
    _say("dense", shape, errors(o[0], ref))
    assert_close(o[0], ref, f"dense {shape}")


def test_dense_bf16_output(absa):
    wl = _random_workload(2, 3, 7, 9, 128, 128, 16, seed=3)
    p = problem(wl, out_bf16=True)
    import torch
    o = absa.dense(p, dev(wl.q), dev(wl.k), dev(wl.v))
    assert o.dtype == torch.bfloat16
    ref = np.stack([O.dense_attention(wl.q[0, h], wl.k[0, h], wl.v[0, h], p.sigma) for h in range(wl.H)])
    # bf16 output adds half an ulp of |o| (<= 2^-9 relative)
    err = np.abs(o.float().cpu().numpy()[0] - ref)
    assert (err <= 1e-2 + 2.0 ** -8 * np.abs(ref)).all()


# ----------------------------------------------------------------------------- attend over oracle lists

@pytest.mark.parametrize("mode", [O.SEL_SIP, O.SEL_TOPK, O.SEL_ALL])
def test_attend_oracle_lists_tiny(absa, mode):
    wl = gen_config(1)
    p = problem(wl)
    res = O.select(wl.q, wl.k, 64, 16, keep32(0.25), mode=mode, seed=0)
    rows, NK = p.rows, p.nk
    count = res.count.astype(np.int32)
    kv = np.zeros((rows, NK), np.int32)
    w = np.zeros((rows, NK), np.float32)
    for r in range(rows):
        kv[r, :count[r]] = res.kv_idx[r]
        w[r, :count[r]] = res.inv_pi[r]
    import torch
    lists = absa.BlockLists(torch.from_numpy(count).cuda(), torch.from_numpy(kv).cuda(),
                            torch.from_numpy(w).cuda())
    o = absa.attend(p, dev(wl.q), dev(wl.k), dev(wl.v), lists).cpu().numpy()
    ref = O.attend_all(wl.q, wl.k, wl.v, 64, 16, count, kv, w, p.sigma)
    _say("attend oracle lists", mode, errors(o, ref))
    assert_close(o, ref, f"attend mode {mode}")


def test_attend_empty_and_invalid_entries(absa):
    import torch
    wl = _random_workload(1, 2, 8, 16, 128, 128, 16, seed=5)  # L = 256, NQ = 2, NK = 16
    p = problem(wl)
    count = torch.tensor([0, 3], dtype=torch.int32).cuda()
    kv = torch.tensor([[0] * 4, [2, 99, 7, 0]], dtype=torch.int32).cuda()  # 99 >= NK: skipped
    w = torch.tensor([[1.0] * 4, [2.0, 1.0, 1.5, 1.0]], dtype=torch.float32).cuda()
    o = absa.attend(p, dev(wl.q), dev(wl.k), dev(wl.v), absa.BlockLists(count, kv, w)).cpu().numpy()
    assert (o[0, 0, :128] == 0).all()
    ref = O.attend_row_block(wl.q, wl.k, wl.v, 0, 1, 128, 16, [2, 7], [2.0, 1.5], p.sigma)
    assert_close(o[0, 0, 128:], ref, "invalid entries")


# ----------------------------------------------------------------------------- exact selection

@pytest.mark.parametrize("seed,collapse", [(0, False), (1, False), (2, True)])
@pytest.mark.parametrize("mode", [O.SEL_SIP, O.SEL_TOPK, O.SEL_ALL])
def test_select_bit_exact_on_integer_inputs(absa, seed, collapse, mode):
    import torch
    wl = gen_exact(seed, groups_collapse=collapse)
    p = problem(wl)
    lists, pi, ws = absa.select(p, dev(wl.q), dev(wl.k), 0.25, clusters=4, kmeans_steps=3,
                                select_scale_log2=1.0, seed=seed + 5, stream_id=3, mode=mode, want_pi=True)
    torch.cuda.synchronize()
    count, kv, w = lists_to_host(lists)
    res = O.select(wl.q, wl.k, 64, 16, 0.25, C=4, Tk=3, alpha=1.0, seed=seed + 5, stream=3, mode=mode,
                   keep_intermediates=True)
    np.testing.assert_array_equal(count, res.count)
    for r in range(p.rows):
        np.testing.assert_array_equal(kv[r, :count[r]], res.kv_idx[r])
        np.testing.assert_array_equal(w[r, :count[r]].view(np.uint32), res.inv_pi[r].view(np.uint32))
    np.testing.assert_array_equal(pi.cpu().numpy().view(np.uint32), res.pi_hat.view(np.uint32))
    # intermediates in the workspace
    offs = absa.workspace_layout(p, 0.25, 4, 3, mode)
    wsn = ws.cpu().numpy()
    NKp = 64
    kbarT = wsn[offs[0]: offs[0] + 2 * 64 * NKp * 4].view(np.float32).reshape(2, 64, NKp)
    np.testing.assert_array_equal(kbarT.transpose(0, 2, 1), res.kbar.astype(np.float32))
    mu = wsn[offs[1]: offs[1] + p.rows * 4 * 64 * 4].view(np.float32).reshape(p.rows, 4, 64)
    np.testing.assert_array_equal(mu, res.mu.astype(np.float32))
    nj = wsn[offs[2]: offs[2] + p.rows * 4 * 4].view(np.int32).reshape(p.rows, 4)
    np.testing.assert_array_equal(nj, res.counts)
    s = wsn[offs[3]: offs[3] + p.rows * 64 * 4].view(np.float32).reshape(p.rows, 64)
    np.testing.assert_array_equal(s, res.scores.astype(np.float32))
    if mode == O.SEL_SIP:
        assert 0 < count.mean() < 64
        assert all((w[r, :count[r]] >= 1).all() for r in range(p.rows))


# ----------------------------------------------------------------------------- general inputs

def _check_selection_and_attend(absa, wl, keep, rows=None, seed=0, mode=O.SEL_SIP, Bk=None, tag=""):
    import torch
    Bk = Bk or wl.kv_block
    p = problem(wl, kv_block=Bk)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists, _, _ = absa.select(p, q, k, keep, seed=seed, mode=mode)
    o = absa.attend(p, q, k, v, lists)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    count, kv, w = lists_to_host(lists)
    all_rows = rows is None
    rows = list(range(p.rows)) if all_rows else rows
    res = O.select(wl.q, wl.k, wl.q_block, Bk, keep32(keep), seed=seed, mode=mode, rows=rows)
    agree = decision_agreement(count, kv, res, p.nk)
    ref = oracle_rows_from_gpu_lists(wl, wl.q_block, Bk, count, kv, w, rows, p.sigma)
    got = gpu_rows(o, wl, wl.q_block, rows)
    g = np.concatenate([got[r] for r in rows])
    rr = np.concatenate([ref[r] for r in rows])
    err = errors(g, rr)
    _say(f"{tag} rows={len(rows)} agreement={agree:.6f} max_abs={err[0]:.3e} rel_l2={err[1]:.3e} "
         f"mean_count={count.mean():.1f}")
    assert agree >= AGREE, f"{tag}: block agreement {agree}"
    assert_close(g, rr, tag)
    # lists are well formed
    assert (count >= 0).all() and (count <= p.nk).all()
    for r in rows:
        c = count[r]
        assert (np.diff(kv[r, :c]) > 0).all() and (kv[r, :c] < p.nk).all() and (w[r, :c] >= 1).all()
    return count, kv, w, o


def test_tiny_workload_end_to_end(absa):
    wl = gen_config(1)
    _check_selection_and_attend(absa, wl, 0.25, tag="tiny")


@pytest.mark.parametrize("T,Hs,Ws,Bq,keep", [
    (1, 1, 1, 64, 0.5),     # L = 1: one query, one KV block of one key
    (1, 1, 17, 64, 0.5),    # L = 17: a second KV block of one key
    (1, 5, 26, 128, 0.3),   # L = 130: a second query block of two queries
])
def test_degenerate_lengths(absa, T, Hs, Ws, Bq, keep):
    wl = _random_workload(2, T, Hs, Ws, 64, Bq, 16, seed=T * 1000 + Hs * 37 + Ws, keep=keep)
    for seed in range(4):  # several draws: kept and dropped blocks, empty lists
        _check_selection_and_attend(absa, wl, keep, seed=seed, tag=f"L={wl.L} seed {seed}")


def test_maximum_kv_blocks(absa):
    # NK = 12288, the most the selection accepts (48 blocks per thread of the SIP kernel)
    wl = _random_workload(2, 48, 64, 64, 128, 128, 16, seed=47, keep=0.08)
    p = problem(wl)
    assert p.nk == 12288
    rows = sample_rows(p.nq, wl.H, 16)
    _check_selection_and_attend(absa, wl, 0.08, rows=rows, tag="NK = 12288 (sampled rows)")


@pytest.mark.parametrize("d,Bq,Bk", [(128, 128, 16), (128, 64, 32), (64, 128, 64), (128, 128, 32),
                                     (128, 128, 64), (64, 64, 16)])
def test_block_size_variants(absa, d, Bq, Bk):
    wl = _random_workload(2, 5, 15, 16, d, Bq, Bk, seed=21, modes=8)  # L = 1200: ragged tails
    _check_selection_and_attend(absa, wl, 0.15, Bk=Bk, tag=f"d{d} Bq{Bq} Bk{Bk}")


@pytest.mark.parametrize("d,Bq", [(128, 128), (128, 64), (64, 128), (64, 64)])
@pytest.mark.parametrize("grid", [(5, 15, 16), (5, 15, 13)])
def test_tile_sized_blocks(absa, d, Bq, grid):
    # 128-key blocks, two 64-key tiles each: L = 1200 ends 48 keys into the last
    # block (its second tile lies wholly past L), L = 975 ends 79 keys into it
    # (the tail falls in the second tile)
    wl = _random_workload(2, *grid, d, Bq, 128, seed=23 + grid[2], modes=8)
    for mode in (O.SEL_SIP, O.SEL_TOPK, O.SEL_ALL):
        _check_selection_and_attend(absa, wl, 0.3, Bk=128, mode=mode, tag=f"d{d} Bq{Bq} Bk128 L={wl.L} mode {mode}")


@pytest.mark.parametrize("mode", [O.SEL_TOPK, O.SEL_ALL])
def test_topk_and_all_modes(absa, mode):
    wl = _random_workload(2, 5, 15, 16, 128, 128, 16, seed=4, modes=8)
    _check_selection_and_attend(absa, wl, 0.1, mode=mode, tag=f"mode {mode}")


def test_all_list_equals_dense_kernel(absa):
    import torch
    wl = _random_workload(2, 5, 15, 16, 128, 128, 16, seed=8, modes=8)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists, _, _ = absa.select(p, q, k, 1.0, mode="all")
    o1 = absa.attend(p, q, k, v, lists)
    o2 = absa.dense(p, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_deterministic(absa):
    import torch
    wl = _random_workload(2, 5, 15, 16, 128, 128, 16, seed=9, modes=8)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    outs = []
    for _ in range(2):
        lists, pi, _ = absa.select(p, q, k, 0.1, seed=7, want_pi=True)
        o = absa.attend(p, q, k, v, lists)
        torch.cuda.synchronize()
        outs.append((lists.count.clone(), lists.kv_idx.clone(), lists.inv_pi.clone(), pi.clone(), o.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_sip_average_approaches_dense(absa):
    """Averaging the single-pass estimate over seeds drives it towards dense attention (the
    estimate's error is mostly variance); top-k truncation at the same budget has a fixed bias."""
    import torch
    wl = gen_config(1)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    dense = absa.dense(p, q, k, v)
    acc = torch.zeros_like(dense)
    errs = []
    n = 64
    for s in range(n):
        lists, _, _ = absa.select(p, q, k, 0.25, seed=s)
        o = absa.attend(p, q, k, v, lists)
        acc += o
        errs.append(float((o - dense).norm() / dense.norm()))
    mean_err = float((acc / n - dense).norm() / dense.norm())
    _say(f"single-pass rel err {np.mean(errs):.4f}, {n}-seed mean rel err {mean_err:.4f}")
    assert mean_err < 0.5 * np.mean(errs)



def test_graph_capture_replays_match_eager(absa):
    # The library allocates nothing, sets no memory and never synchronises, so a step of selection
    # and attention can be captured into a graph; every replay, with eager work clobbering the
    # outputs in between, must reproduce the eager result bit for bit.
    import torch
    wl = _random_workload(2, 5, 15, 16, 128, 128, 16, seed=11, modes=8)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists = absa.alloc_lists(p)
    ws = torch.empty(absa.select_workspace_bytes(p, 0.1), dtype=torch.uint8, device="cuda")
    o = torch.empty((p.B, p.H, p.L, p.d), dtype=torch.float32, device="cuda")

    def step():
        absa.select(p, q, k, 0.1, seed=5, lists=lists, workspace=ws)
        absa.attend(p, q, k, v, lists, out=o)

    def clobber():
        o.zero_()
        lists.count.zero_()
        lists.kv_idx.zero_()
        lists.inv_pi.zero_()

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

# ----------------------------------------------------------------------------- full-size workloads

def test_wan13b_480p_full(absa):
    wl = gen_config(2)
    p = problem(wl)
    rows = sample_rows(p.nq, wl.H, 48)
    _check_selection_and_attend(absa, wl, 0.10, rows=rows, tag="Wan2.1-1.3B 480p (sampled rows)")


@pytest.mark.parametrize("keep", [0.08, 0.095, 0.11])
def test_wan14b_720p_full(absa, keep):
    wl = _wan14b()
    p = problem(wl)
    rows = sample_rows(p.nq, wl.H, 32)
    _check_selection_and_attend(absa, wl, keep, rows=rows, tag=f"Wan2.1-14B 720p keep {keep}")


def test_hunyuan_720p_full(absa):
    wl = gen_config(4)
    p = problem(wl)
    rows = sample_rows(p.nq, wl.H, 32)
    _check_selection_and_attend(absa, wl, 0.08, rows=rows, tag="HunyuanVideo 720p Bk16")
    _check_selection_and_attend(absa, wl, 0.08, rows=rows, Bk=32, tag="HunyuanVideo 720p Bk32")


_WAN14 = {}


def _wan14b():
    if "wl" not in _WAN14:
        _WAN14["wl"] = gen_config(3)
    return _WAN14["wl"]
