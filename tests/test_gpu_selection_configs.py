"""GPU parity of the selection knobs and of the prior-art arm against the fp64 oracle.

* Bit-exact: absa_select with C in {1, 2, 4, 8} clusters and Tk in {1, 2, 3} k-means steps, in
  SIP and TOPK modes, on the second integer workload (tests/exact_family.py), whose k-means keeps
  moving after its first step in a share of the blocks: lists, probabilities and the workspace's
  intermediates equal the oracle's bit for bit.
* Agreement: the same knobs on the tiny workload (every row) and the Wan2.1-14B 720p workload
  (sampled rows, head tails included): >= 99.9% of block decisions, and the attention outputs
  within max-abs 1e-2 / rel-L2 5e-3 of the oracle fed the GPU's lists.
* The prior-art arm of the AB-Attention page's bottleneck section (one mean query per block, top-k
  truncation, tile-sized KV blocks) end to end at the 720p shape.
* Dense attention at the 720p shape on sampled rows, the 80-query tail block included.
* The seed average of the SIP estimate against its exact expectation (every Poisson subset
  enumerated by the oracle), within a CLT bound."""
import sys

import numpy as np
import pytest

import oracle as O
from exact_family import gen_exact_family
from gpu_helpers import (AGREE, assert_close, assert_selection_bit_exact, decision_agreement, dev, errors,
                         gpu_rows, keep32, lists_to_host, oracle_rows_from_gpu_lists, problem, sample_rows)
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


_WL = {}


def _wan14b():
    if "wan" not in _WL:
        _WL["wan"] = gen_config(3)
    return _WL["wan"]


def _dev_qkv(wl):
    key = ("dev", id(wl))
    if key not in _WL:
        _WL[key] = (dev(wl.q), dev(wl.k), dev(wl.v))
    return _WL[key]


# ----------------------------------------------------------------------------- bit-exact knobs

@pytest.mark.parametrize("mode", [O.SEL_SIP, O.SEL_TOPK])
@pytest.mark.parametrize("C,Tk", [(1, 1), (1, 3), (2, 1), (2, 2), (2, 3), (4, 1), (4, 2), (4, 3),
                                  (8, 1), (8, 2), (8, 3)])
def test_select_bit_exact_integer_family(absa, C, Tk, mode):
    wl = gen_exact_family(C * 10 + Tk, C, Tk)
    count, _, _ = assert_selection_bit_exact(absa, wl, C, Tk, mode, seed=C + 7 * Tk)
    _say(f"integer family C={C} Tk={Tk} mode {mode}: bit-exact, {wl.extra['moved_blocks']} of 32 blocks "
         f"move after step 1, mean kept {count.mean():.2f}")
    if Tk >= 2 and C >= 2:
        assert wl.extra["moved_blocks"] >= 8


# ----------------------------------------------------------------------------- agreement on general inputs

def _check(absa, wl, keep, rows, C, Tk, mode, Bk=None, tag=""):
    import torch
    Bk = Bk or wl.kv_block
    p = problem(wl, kv_block=Bk)
    q, k, v = _dev_qkv(wl)
    lists, _, _ = absa.select(p, q, k, keep, clusters=C, kmeans_steps=Tk, seed=11, mode=mode)
    o = absa.attend(p, q, k, v, lists)
    torch.cuda.synchronize()
    count, kv, w = lists_to_host(lists)
    rows = list(range(p.rows)) if rows is None else rows
    res = O.select(wl.q, wl.k, wl.q_block, Bk, keep32(keep), C=C, Tk=Tk, seed=11, mode=mode, rows=rows)
    agree = decision_agreement(count, kv, res, p.nk)
    ref = oracle_rows_from_gpu_lists(wl, wl.q_block, Bk, count, kv, w, rows, p.sigma)
    got = gpu_rows(o.cpu().numpy(), wl, wl.q_block, rows)
    g = np.concatenate([got[r] for r in rows])
    rr = np.concatenate([ref[r] for r in rows])
    err = errors(g, rr)
    _say(f"{tag} C={C} Tk={Tk} mode {mode} Bk {Bk}: rows={len(rows)} agreement={agree:.6f} "
         f"max_abs={err[0]:.3e} rel_l2={err[1]:.3e} mean_count={count.mean():.1f}")
    assert agree >= AGREE, f"{tag}: block agreement {agree}"
    assert_close(g, rr, tag)


KNOBS = [(1, 3), (2, 3), (8, 3), (4, 1), (4, 2)]


@pytest.mark.parametrize("mode", [O.SEL_SIP, O.SEL_TOPK])
@pytest.mark.parametrize("C,Tk", KNOBS)
def test_select_knobs_tiny(absa, C, Tk, mode):
    wl = gen_config(1)
    _check(absa, wl, 0.25, None, C, Tk, mode, tag="tiny")


@pytest.mark.parametrize("mode", [O.SEL_SIP, O.SEL_TOPK])
@pytest.mark.parametrize("C,Tk", KNOBS)
def test_select_knobs_wan14b_720p(absa, C, Tk, mode):
    wl = _wan14b()
    p = problem(wl)
    rows = sample_rows(p.nq, wl.H, 16, seed=100 + C * 10 + Tk)
    _check(absa, wl, 0.095, rows, C, Tk, mode, tag="Wan2.1-14B 720p")


@pytest.mark.parametrize("Bk", [64, 128])
def test_prior_art_arm_wan14b_720p(absa, Bk):
    # one mean query per query block (C = 1), top-k truncation, KV blocks of one
    # 64-key tile or of a whole 128 x 128 tile
    wl = _wan14b()
    p = problem(wl, kv_block=Bk)
    rows = sample_rows(p.nq, wl.H, 24, seed=321)
    _check(absa, wl, 0.10, rows, 1, 3, O.SEL_TOPK, Bk=Bk, tag="prior-art arm 720p")


# ----------------------------------------------------------------------------- dense at the 720p shape

def test_dense_wan14b_720p_sampled_rows(absa):
    import torch
    wl = _wan14b()
    p = problem(wl)
    q, k, v = _dev_qkv(wl)
    o = absa.dense(p, q, k, v)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    rows = sample_rows(p.nq, wl.H, 12, seed=55, tails=4)
    assert any(r % p.nq == p.nq - 1 for r in rows)          # the 80-query tail block
    got = gpu_rows(o, wl, wl.q_block, rows)
    g, rr = [], []
    for r in rows:
        bh, i = divmod(int(r), p.nq)
        t0, t1 = i * 128, min(wl.L, (i + 1) * 128)
        rr.append(O.dense_rows(wl.q, wl.k, wl.v, bh, t0, t1, p.sigma))
        g.append(got[r])
    err = assert_close(np.concatenate(g), np.concatenate(rr), "dense 720p sampled rows")
    _say(f"dense 720p: rows={len(rows)} max_abs={err[0]:.3e} rel_l2={err[1]:.3e}")


# ----------------------------------------------------------------------------- seed average

def test_sip_seed_average_matches_exact_expectation(absa):
    """Over seeds, the GPU's SIP estimate averages to the exact expectation of the estimator
    (every Poisson subset of the row's uncertain blocks enumerated by the oracle, with the fp32
    probabilities and weights).  Per element, |mean - E[o]| <= 6 sqrt(Var[o] / S) + 1e-2, the
    last term for the bf16 arithmetic of a single estimate; the ratio's expectation is not dense
    attention (only its numerator and denominator are unbiased), so E[o] is the reference."""
    import torch
    q, k, v = (bf16_round(x) for x in gen_fourier_heads(1, 16, 16, 64, 4, 0.3, False, 5, [0]))
    wl = Workload(q=q[None], k=k[None], v=v[None], B=1, H=1, L=256, d=64, T=1, Hs=16, Ws=16, q_block=64,
                  kv_block=16, keep=0.25)
    p = problem(wl)
    qd, kd, vd = dev(wl.q), dev(wl.k), dev(wl.v)
    rows = [1, 2]
    _, pi, _ = absa.select(p, qd, kd, 0.25, seed=0, want_pi=True)
    pi = pi.cpu().numpy()
    # the sampler's own probabilities define the estimator's distribution; they agree with the
    # oracle's to the selection's arithmetic (split-bf16 products, fp32 sums)
    res = O.select(wl.q, wl.k, 64, 16, keep32(0.25), rows=rows)
    np.testing.assert_allclose(pi[rows], res.pi_hat, rtol=1e-4, atol=1e-6)
    S = 512
    acc = torch.zeros((1, 1, 256, 64), dtype=torch.float64, device="cuda")
    lists = absa.alloc_lists(p)
    out = torch.empty((1, 1, 256, 64), dtype=torch.float32, device="cuda")
    for s in range(S):
        absa.select(p, qd, kd, 0.25, seed=1000 + s, lists=lists)
        absa.attend(p, qd, kd, vd, lists, out=out)
        acc += out.double()
    mean = (acc / S).cpu().numpy()[0, 0]
    for r_i, r in enumerate(rows):
        m1, m2 = O.sip_output_moments(wl.q[0, 0, r * 64:(r + 1) * 64], wl.k[0, 0], wl.v[0, 0], pi[r], 16, p.sigma)
        sd = np.sqrt(np.maximum(m2 - m1 * m1, 0.0) / S)
        dev_ = np.abs(mean[r * 64:(r + 1) * 64] - m1)
        z = dev_ / np.maximum(sd, 1e-12)
        _say(f"row {r}: max |mean - E[o]| {dev_.max():.3e}, sd of the mean {sd.mean():.3e}, max z {z.max():.2f}, "
             f"rms z {np.sqrt((z ** 2).mean()):.2f}")
        assert np.all(dev_ <= 6.0 * sd + 1e-2)


# ----------------------------------------------------------------------------- sampler at large NK

@pytest.mark.parametrize("grid", [(16, 40, 150), (14, 40, 200), (18, 40, 200), (22, 40, 200)])
def test_sampler_large_block_counts(absa, grid):
    """NK = 6000, 7000 (two waves per list, 12- and 16-block chunks), 9000 and 11000 (four waves,
    12-block chunks) at Bk = 16.  On sampled rows, given the scores the selection wrote to its
    workspace, the lists follow the sampling definition exactly: top-k keeps the k* highest scores
    (ties to the lower index); SIP keeps b iff u_b < pi_b for the oracle's Philox uniforms and the
    kernel's fp32 pi, with weights fp32(1 / pi), and pi equals the oracle's capping of the same
    scores to the fp32 rounding of its sums.  Decisions also agree with the oracle's own selection,
    and the outputs with the oracle fed the GPU's lists."""
    import torch
    T, Hs, Ws = grid
    q, k, v = (bf16_round(x) for x in gen_fourier_heads(T, Hs, Ws, 128, 8, 0.3, False, 60 + T, [0, 1]))
    L = T * Hs * Ws
    sh = (1, 2, L, 128)
    wl = Workload(q=q.reshape(sh), k=k.reshape(sh), v=v.reshape(sh), B=1, H=2, L=L, d=128, T=T, Hs=Hs, Ws=Ws,
                  q_block=128, kv_block=16, keep=0.08)
    p = problem(wl)
    NK = p.nk
    NKs = -(-NK // 4) * 4
    keep = 0.08
    n_star = keep32(keep) * NK
    rows = sample_rows(p.nq, wl.H, 12, seed=70 + T)
    qd, kd, vd = dev(wl.q), dev(wl.k), dev(wl.v)
    for mode in (O.SEL_SIP, O.SEL_TOPK):
        seed, stream_id = 17, 2
        lists, pi, ws = absa.select(p, qd, kd, keep, seed=seed, stream_id=stream_id, mode=mode, want_pi=True)
        o = absa.attend(p, qd, kd, vd, lists)
        torch.cuda.synchronize()
        count, kv, w = lists_to_host(lists)
        pi = pi.cpu().numpy()
        offs = absa.workspace_layout(p, keep, mode=mode)
        s_all = ws.cpu().numpy()[offs[3]: offs[3] + p.rows * NKs * 4].view(np.float32).reshape(p.rows, NKs)
        assert not s_all[:, NK:].any()
        max_rel = 0.0
        for r in rows:
            bh, i = divmod(int(r), p.nq)
            s = s_all[r, :NK].astype(np.float64)
            got = kv[r, :count[r]]
            if mode == O.SEL_TOPK:
                ref, _, _ = O.select_row(s, n_star, O.SEL_TOPK, seed, stream_id, bh, i)
                np.testing.assert_array_equal(got, ref)
                assert (w[r, :count[r]] == 1.0).all()
                np.testing.assert_array_equal(np.nonzero(pi[r])[0], ref)
            else:
                u = O.sip_uniforms(seed, stream_id, bh, i, NK)
                np.testing.assert_array_equal(got, np.nonzero(u < pi[r].astype(np.float64))[0])
                inv = (np.float32(1.0) / pi[r, got]).astype(np.float32)
                np.testing.assert_array_equal(w[r, :count[r]].view(np.uint32), inv.view(np.uint32))
                ref_pi = O.sip_inclusion(s, n_star)
                rel = np.abs(pi[r] - ref_pi) / np.maximum(ref_pi, 1e-30)
                max_rel = max(max_rel, float(rel[ref_pi > 0].max()))
                assert ((pi[r] > 0) == (ref_pi > 0)).all()
                assert rel[ref_pi > 0].max() <= 1e-4
        res = O.select(wl.q, wl.k, 128, 16, keep32(keep), seed=seed, stream=stream_id, mode=mode, rows=rows)
        agree = decision_agreement(count, kv, res, NK)
        ref_o = oracle_rows_from_gpu_lists(wl, 128, 16, count, kv, w, rows, p.sigma)
        g = gpu_rows(o.cpu().numpy(), wl, 128, rows)
        err = assert_close(np.concatenate([g[r] for r in rows]), np.concatenate([ref_o[r] for r in rows]),
                           f"NK={NK} mode {mode}")
        _say(f"NK={NK} mode {mode}: rows={len(rows)} lists follow the definition on the kernel's scores "
             f"(max rel pi diff {max_rel:.2e}), agreement={agree:.6f} max_abs={err[0]:.3e} rel_l2={err[1]:.3e} "
             f"mean_count={count.mean():.1f}")
        assert agree >= AGREE


# ----------------------------------------------------------------------------- measurement entry point

def test_select_profile_gives_the_same_lists(absa):
    """absa_select_profile: the lists of absa_select, bit for bit, and five positive kernel times."""
    import torch
    wl = gen_config(1)
    p = problem(wl)
    q, k = dev(wl.q), dev(wl.k)
    ref, _, _ = absa.select(p, q, k, 0.25, seed=3)
    got, times = absa.select_profile(p, q, k, 0.25, seed=3)
    torch.cuda.synchronize()
    for a, b in zip((got.count, got.kv_idx, got.inv_pi), (ref.count, ref.kv_idx, ref.inv_pi)):
        assert torch.equal(a, b)
    assert list(times) == list(absa.SELECT_KERNELS)
    assert all(t > 0.0 for t in times.values())
