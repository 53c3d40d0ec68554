"""Pins of the fp64 oracle against things other than itself: closed forms, library routines
that compute the same quantity, brute force, and identities the method must satisfy.

Each test names the oracle step it pins (S1..S6, as in the oracle's header)."""
import itertools
import math

import numpy as np
import pytest
import scipy.cluster.vq
import scipy.special
import torch

import oracle as O
from golden_figures import page_figure
from workloads import CONFIGS, gen_config, gen_exact, gen_micro


# ----------------------------------------------------------------------------- dense ([XA] formula)

def test_dense_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((37, 24)) for _ in range(3))
    sigma = 0.31
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], scale=sigma)[0, 0].numpy()
    np.testing.assert_allclose(O.dense_attention(q, k, v, sigma), ref, rtol=1e-12, atol=1e-13)


def test_dense_rows_sum_to_one_and_uniform_case():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((20, 8)), rng.standard_normal((50, 8))
    P = O.dense_attention(q, k, np.eye(50), 0.7)  # V = I returns the attention matrix
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (P >= 0).all()
    v = rng.standard_normal((50, 8))
    # q = 0: every key gets weight 1/L, so the output is the mean value row.
    np.testing.assert_allclose(O.dense_attention(np.zeros((3, 8)), k, v, 1.0),
                               np.tile(v.mean(axis=0), (3, 1)), rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- S1

def test_kv_block_means_tail_by_brute_force():
    rng = np.random.default_rng(2)
    k = rng.integers(-5, 6, size=(37, 3)).astype(np.float64)
    kb = O.kv_block_means(k, 8)
    assert kb.shape == (5, 3)
    for b in range(5):
        rows = [t for t in range(37) if t // 8 == b]
        for c in range(3):
            assert kb[b, c] == pytest.approx(sum(k[t, c] for t in rows) / len(rows), abs=1e-15)
    assert len([t for t in range(37) if t // 8 == 4]) == 5  # the partial block has 5 keys


# ----------------------------------------------------------------------------- S2

@pytest.mark.parametrize("seed", range(6))
def test_kmeans_equals_scipy_kmeans2(seed):
    rng = np.random.default_rng(seed)
    n, d, C, Tk = 64, 16, 4, 3
    X = np.concatenate([rng.standard_normal((16, d)) + 3 * rng.standard_normal(d) for _ in range(4)])
    X = X[rng.permutation(n)]
    mu, counts, labels = O.ibcs_kmeans(X, C, Tk)
    init = np.stack([X[(j * n) // C] for j in range(C)])
    with np.errstate(all="ignore"):
        import warnings
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            ref_mu, ref_lab = scipy.cluster.vq.kmeans2(X, init.copy(), iter=Tk, minit="matrix",
                                                       missing="warn")
    np.testing.assert_allclose(mu, ref_mu, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(labels, ref_lab)
    np.testing.assert_array_equal(counts, np.bincount(ref_lab, minlength=C))


def test_kmeans_empty_cluster_keeps_centroid_like_scipy():
    # Two identical initial members: cluster 1 ties with cluster 0 on every point and the
    # lowest index wins, so cluster 1 is empty and must keep its initial centroid.
    X = np.array([[0.0, 0.0], [5.0, 5.0], [0.0, 0.0], [6.0, 5.0]])
    mu, counts, _ = O.ibcs_kmeans(X, 2, 2)
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        ref_mu, _ = scipy.cluster.vq.kmeans2(X, np.stack([X[0], X[2]]), iter=2, minit="matrix",
                                             missing="warn")
    np.testing.assert_allclose(mu, ref_mu)
    assert counts.tolist() == [2, 2]  # step 2 moves the zeros onto the kept centroid
    mu1, counts1, _ = O.ibcs_kmeans(X, 2, 1)
    assert counts1.tolist() == [4, 0]
    np.testing.assert_array_equal(mu1[1], X[2])  # empty after step 1: centroid unchanged
    np.testing.assert_allclose(mu1[0], X.mean(axis=0))


def test_kmeans_closed_forms():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((40, 6))
    mu, counts, _ = O.ibcs_kmeans(X, 1, 3)  # one cluster: the block's mean query
    np.testing.assert_allclose(mu[0], X.mean(axis=0), rtol=1e-14)
    assert counts.tolist() == [40]
    mu, counts, labels = O.ibcs_kmeans(X, 40, 2)  # C = n: every query is its own centroid
    np.testing.assert_allclose(mu, X)
    assert counts.tolist() == [1] * 40 and labels.tolist() == list(range(40))


def test_kmeans_objective_non_increasing():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((128, 32)) * np.linspace(0.2, 3.0, 32)
    prev = np.inf
    for Tk in range(1, 8):
        mu, _, labels = O.ibcs_kmeans(X, 4, Tk)
        J = ((X - mu[labels]) ** 2).sum()
        assert J <= prev + 1e-9
        prev = J


# ----------------------------------------------------------------------------- S3

def test_scores_degenerate_case_is_softmax():
    # Query block of one query, KV blocks of one key, one cluster: s = softmax(sigma q . K).
    rng = np.random.default_rng(5)
    q = rng.standard_normal(16)
    K = rng.standard_normal((30, 16))
    sigma = 0.4
    mu, counts, _ = O.ibcs_kmeans(q[None], 1, 3)
    s = O.ibcs_scores(mu, counts, O.kv_block_means(K, 1), np.ones(30), sigma * math.log2(math.e))
    np.testing.assert_allclose(s, scipy.special.softmax(sigma * (K @ q)), rtol=1e-12, atol=1e-15)


def test_scores_hand_worked_example():
    """Small example derived by hand from S1-S4.

    Queries (1,0),(1,0),(0,1),(0,1), C=2, Tk=1: init at members 0 and 2, clusters {0,1},{2,3},
    centroids (1,0),(0,1), counts (2,2).  Keys (1,0),(1,0) | (0,1),(0,3) | (1,1) with KV block 2
    (last block holds one key): means (1,0),(0,2),(1,1), valid counts (2,2,1).  alpha = 1:
    centroid 0 logits (1,0,1): e = (2, 2*2^-1, 1) = (2,1,1), Z = 4 -> (1/2, 1/4, 1/4);
    centroid 1 logits (0,2,1): e = (2*2^-2, 2, 2^-1) = (1/2, 2, 1/2), Z = 3 -> (1/6, 2/3, 1/6);
    s = (1/3, 11/24, 5/24).
    keep 1/2 (n* = 1.5): no cap (1.5 s < 1), pi = 1.5 s = (1/2, 11/16, 5/16).
    keep 0.8 (n* = 2.4): 2.4 * 11/24 >= 1 caps block 1; then R = 1.4, S_U = 13/24 and
    pi = (1.4*8/13, 1, 7/13).  TOPK at n* = 1.5 keeps k* = 2 blocks: {0, 1}.
    """
    X = np.array([[1.0, 0], [1, 0], [0, 1], [0, 1]])
    K = np.array([[1.0, 0], [1, 0], [0, 1], [0, 3], [1, 1]])
    mu, counts, _ = O.ibcs_kmeans(X, 2, 1)
    np.testing.assert_array_equal(mu, [[1, 0], [0, 1]])
    assert counts.tolist() == [2, 2]
    kb = O.kv_block_means(K, 2)
    np.testing.assert_array_equal(kb, [[1, 0], [0, 2], [1, 1]])
    s = O.ibcs_scores(mu, counts, kb, np.array([2, 2, 1]), 1.0)
    np.testing.assert_allclose(s, [1 / 3, 11 / 24, 5 / 24], rtol=1e-15)
    np.testing.assert_allclose(O.sip_inclusion(s, 1.5), [0.5, 11 / 16, 5 / 16], rtol=1e-15)
    np.testing.assert_allclose(O.sip_inclusion(s, 2.4), [1.4 * 8 / 13, 1.0, 7 / 13], rtol=1e-14)
    idx, w, ph = O.select_row(s, 1.5, O.SEL_TOPK, 0, 0, 0, 0)
    assert idx.tolist() == [0, 1] and w.tolist() == [1, 1] and ph.tolist() == [1, 1, 0]


def test_scores_floor_drops_far_blocks():
    mu = np.array([[1.0]])
    kb = np.array([[0.0], [-63.0], [-65.0]])
    s = O.ibcs_scores(mu, np.array([3]), kb, np.ones(3), 1.0)
    assert s[2] == 0.0 and s[1] > 0.0
    np.testing.assert_allclose(s.sum(), 1.0, rtol=1e-15)


def test_scores_sum_to_one_on_workload():
    wl = gen_config(1)
    res = O.select(wl.q, wl.k, 64, 16, 0.25, rows=[0, 5, 17, 31], keep_intermediates=True)
    np.testing.assert_allclose(res.scores.sum(axis=1), 1.0, rtol=1e-12)


# ----------------------------------------------------------------------------- S4

@pytest.mark.parametrize("seed", range(5))
def test_capping_equals_bisection(seed):
    rng = np.random.default_rng(seed)
    s = rng.pareto(1.2, size=500)
    s[rng.integers(0, 500, 30)] = 0.0
    s /= s.sum()
    for n_star in (1.0, 12.5, 50.0, 200.0, 469.0, 470.0, 499.0, 500.0):
        pi = O.sip_inclusion(s, n_star)
        ref = O.bisection_inclusion(s, n_star)
        np.testing.assert_allclose(pi, ref, rtol=1e-9, atol=1e-12)
        assert (pi <= 1.0).all() and (pi >= 0).all()
        expect = 500 if n_star >= 500 else min(n_star, (s > 0).sum())  # n* >= NK: pi = 1 everywhere
        np.testing.assert_allclose(pi.sum(), expect, rtol=1e-12)
        free = (pi < 1.0) & (s > 0)
        if free.any():
            ratio = pi[free] / s[free]
            np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)
            assert (s[pi == 1.0] >= s[free].max()).all()  # capped blocks are the largest


def test_capping_budget_beyond_blocks():
    s = np.array([0.5, 0.5, 0.0])
    np.testing.assert_array_equal(O.sip_inclusion(s, 3.0), [1, 1, 1])
    np.testing.assert_array_equal(O.sip_inclusion(s, 2.5), [1, 1, 0])


# ----------------------------------------------------------------------------- S5

def test_philox_all_zero_block():
    # Counter 0, key 0: the first block of the Philox4x32-10 stream.
    out = O.philox4x32_10(np.zeros(4, np.uint32), np.zeros(2, np.uint32))
    assert [int(x) for x in out] == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]


def test_uniforms_are_uniform():
    u = np.concatenate([O.sip_uniforms(3, 1, bh, i, 4096) for bh in range(4) for i in range(8)])
    assert (u >= 0).all() and (u < 1).all()
    assert np.all((u * 2 ** 24) == np.floor(u * 2 ** 24))  # 24-bit grid
    hist = np.histogram(u, bins=32, range=(0, 1))[0]
    exp = u.size / 32
    chi2 = ((hist - exp) ** 2 / exp).sum()
    assert chi2 < 70.0  # 31 dof: p < 1e-4 beyond this
    # distinct rows get distinct streams
    assert not np.array_equal(O.sip_uniforms(3, 1, 0, 0, 64), O.sip_uniforms(3, 1, 0, 1, 64))
    assert not np.array_equal(O.sip_uniforms(3, 1, 0, 0, 64), O.sip_uniforms(4, 1, 0, 0, 64))
    assert not np.array_equal(O.sip_uniforms(3, 1, 0, 0, 64), O.sip_uniforms(3, 2, 0, 0, 64))


def test_inclusion_frequencies_match_pi():
    s = np.random.default_rng(9).pareto(1.0, 40)
    s /= s.sum()
    n_star = 8.0
    hits = np.zeros(40)
    N = 4000
    pi_hat = None
    for seed in range(N):
        idx, w, pi_hat = O.select_row(s, n_star, O.SEL_SIP, seed, 0, 0, 0)
        hits[idx] += 1
        np.testing.assert_array_equal(w, (1.0 / pi_hat[idx].astype(np.float64)).astype(np.float32))
    p = pi_hat.astype(np.float64)
    sd = np.sqrt(p * (1 - p) / N)
    assert np.all(np.abs(hits / N - p) <= 5 * sd + 1e-12)


def test_topk_invariants():
    rng = np.random.default_rng(11)
    s = rng.integers(0, 6, size=300).astype(np.float64)  # many ties
    for n_star in (0.2, 0.5, 7.49, 7.5, 100.0, 299.6, 400.0):
        idx, w, ph = O.select_row(s, n_star, O.SEL_TOPK, 0, 0, 0, 0)
        kstar = min(300, int(math.floor(n_star + 0.5)))
        assert len(idx) == kstar and (np.diff(idx) > 0).all() and (w == 1).all()
        kept = np.zeros(300, bool)
        kept[idx] = True
        if kstar and kstar < 300:
            assert s[kept].min() >= s[~kept].max()
            thr = s[kept].min()
            # among blocks tied at the threshold, the kept ones have the lowest indices
            tied = np.nonzero(s == thr)[0]
            kt = tied[kept[tied]]
            assert (kt == tied[: len(kt)]).all()


# ----------------------------------------------------------------------------- S6

def _micro_setup():
    wl = gen_micro()
    q, k, v = (a[0, 0].astype(np.float64) for a in (wl.q, wl.k, wl.v))
    res = O.select(wl.q, wl.k, 64, 16, 0.25, C=2, Tk=2, rows=[1], keep_intermediates=True)
    return wl, q, k, v, res.scores[0]


def test_enumeration_horvitz_thompson_identity():
    """E over every Poisson subset of num and den equals the dense num and den."""
    wl, q, k, v, s = _micro_setup()
    NK, sigma = 16, 1.0 / 4.0
    pi = O.sip_inclusion(s, 0.25 * NK)
    qb = q[64:128]
    shift = (sigma * qb @ k.T).max(axis=1)
    dense_num, dense_den = O.estimator_num_den(qb, k, v, range(NK), np.ones(NK), 16, sigma, shift)
    certain = [b for b in range(NK) if pi[b] == 1.0]
    U = [b for b in range(NK) if 0.0 < pi[b] < 1.0]
    assert 4 <= len(U) <= 16
    e_num = np.zeros_like(dense_num)
    e_den = np.zeros_like(dense_den)
    tot_p = 0.0
    for mask in itertools.product([0, 1], repeat=len(U)):
        S = certain + [b for b, m in zip(U, mask) if m]
        p = np.prod([pi[b] if m else 1.0 - pi[b] for b, m in zip(U, mask)])
        tot_p += p
        if S:
            num, den = O.estimator_num_den(qb, k, v, S, [1.0 / pi[b] for b in S], 16, sigma, shift)
            e_num += p * num
            e_den += p * den
    assert tot_p == pytest.approx(1.0, abs=1e-12)
    np.testing.assert_allclose(e_num, dense_num, rtol=1e-11, atol=1e-12 * np.abs(dense_num).max())
    np.testing.assert_allclose(e_den, dense_den, rtol=1e-12)


def test_all_blocks_equals_dense():
    wl = gen_config(1)
    q, k, v = wl.q, wl.k, wl.v
    sigma = 1.0 / 8.0
    res = O.select(q, k, 64, 16, 0.25, mode=O.SEL_ALL, rows=[3, 20])
    for r_i, r in enumerate(res.rows):
        bh, i = divmod(int(r), 16)
        out = O.attend_row_block(q, k, v, bh, i, 64, 16, res.kv_idx[r_i], res.inv_pi[r_i], sigma)
        ref = O.dense_rows(q, k, v, bh, 64 * i, 64 * i + 64, sigma)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    # keep = 1 in SIP mode: every pi is 1 and the estimate is dense attention
    res = O.select(q, k, 64, 16, 1.0, mode=O.SEL_SIP, rows=[7])
    assert res.count[0] == 64 and (res.inv_pi[0] == 1).all()


def test_estimator_brute_force_with_tails():
    """S6 against per-query pure-Python loops on L not divisible by either block size."""
    rng = np.random.default_rng(12)
    L, d, Bq, Bk = 45, 4, 16, 8
    q = rng.standard_normal((1, 1, L, d))
    k = rng.standard_normal((1, 1, L, d))
    v = rng.standard_normal((1, 1, L, d))
    kept, w = [1, 3, 5], [2.0, 1.25, 4.0]  # block 5 holds keys 40..44 only
    sigma = 0.6
    out = O.attend_row_block(q, k, v, 0, 2, Bq, Bk, kept, w, sigma)  # queries 32..44
    assert out.shape == (13, d)
    for t in range(32, 45):
        num = [0.0] * d
        den = 0.0
        for b, wb in zip(kept, w):
            for key in range(b * Bk, min(L, (b + 1) * Bk)):
                a = sigma * sum(q[0, 0, t, c] * k[0, 0, key, c] for c in range(d))
                e = wb * math.exp(a)
                den += e
                for c in range(d):
                    num[c] += e * v[0, 0, key, c]
        np.testing.assert_allclose(out[t - 32], np.array(num) / den, rtol=1e-12)
    empty = O.attend_row_block(q, k, v, 0, 0, Bq, Bk, [], [], sigma)
    assert (empty == 0).all()


# ----------------------------------------------------------------------------- EXACT workload

@pytest.mark.parametrize("seed", [0, 1])
def test_exact_workload_closed_form(seed):
    """On the integer workload the k-means recovers the group centres and the scores equal the
    closed form s_b = sum_j 2^(a_j[b] - E_j - 2), E_j = log2 sum_b 2^a_j[b]; every
    intermediate is exactly representable in fp32."""
    wl = gen_exact(seed)
    res = O.select(wl.q, wl.k, 64, 16, 0.25, C=4, Tk=3, alpha=1.0, keep_intermediates=True)
    NQ = 16
    for r in range(len(res.rows)):
        bh, i = divmod(r, NQ)
        X = wl.q[0, bh, 64 * i: 64 * i + 64].astype(np.float64)
        centres = np.stack([X[16 * j:16 * j + 16].mean(axis=0) for j in range(4)])
        np.testing.assert_array_equal(res.mu[r], centres)
        assert res.counts[r].tolist() == [16] * 4
        s_cf = np.zeros(64)
        for j in range(4):
            a = centres[j]
            E = math.log2(np.exp2(a[a > -64]).sum())
            assert E == int(E)
            s_cf += np.where(a > -64, np.exp2(a - E - 2), 0.0)
        np.testing.assert_array_equal(res.scores[r], s_cf)
        assert np.array_equal(res.scores[r].astype(np.float32).astype(np.float64), res.scores[r])
        pi = O.sip_inclusion(res.scores[r], 16.0)
        assert 0 < (pi == 1).sum() or (pi < 1).all()
    np.testing.assert_array_equal(res.kbar[:, :, :], np.broadcast_to(np.eye(64), (2, 64, 64)))


# ----------------------------------------------------------------------------- per-cluster lists (C1-C4)

def test_cluster_scores_mixture_and_normalisation():
    rng = np.random.default_rng(31)
    C, NK, d = 4, 37, 16
    mu = rng.standard_normal((C, d))
    counts = np.array([5, 0, 9, 2])
    kbar = rng.standard_normal((NK, d))
    nk = np.full(NK, 16.0)
    nk[-1] = 7.0
    s = O.cluster_scores(mu, counts, kbar, nk, 0.9)
    np.testing.assert_allclose(s.sum(axis=1), [1, 0, 1, 1], rtol=1e-13)
    mix = (counts[:, None] / counts.sum() * s).sum(axis=0)
    np.testing.assert_allclose(mix, O.ibcs_scores(mu, counts, kbar, nk, 0.9), rtol=1e-12, atol=1e-15)
    # a one-member cluster at a block mean: that block has the largest score
    mu1 = kbar[[3]] * 5
    s1 = O.cluster_scores(mu1, np.array([1]), kbar, np.full(NK, 16.0), 1.0)
    assert np.argmax(s1[0]) == np.argmax(kbar @ mu1[0])


def test_one_cluster_equals_shared_selection():
    wl = gen_micro(3)
    for mode in (O.SEL_SIP, O.SEL_TOPK):
        shared = O.select(wl.q, wl.k, wl.q_block, wl.kv_block, 0.3, C=1, mode=mode, seed=5, stream=2)
        per = O.select_clusters(wl.q, wl.k, wl.q_block, wl.kv_block, 0.3, C=1, mode=mode, seed=5, stream=2)
        for r_i in range(len(shared.rows)):
            idx, w, ph = per.lists[r_i][0]
            np.testing.assert_array_equal(idx, shared.kv_idx[r_i])
            np.testing.assert_array_equal(w, shared.inv_pi[r_i])
            np.testing.assert_array_equal(ph, shared.pi_hat[r_i])


def test_cluster_streams_differ_and_union_weights():
    u0 = O.cluster_uniforms(7, 0, 3, 5, 0, 4, 64)
    u1 = O.cluster_uniforms(7, 0, 3, 5, 1, 4, 64)
    assert not np.array_equal(u0, u1)
    np.testing.assert_array_equal(O.cluster_uniforms(7, 0, 3, 20, 1, 4, 64), O.sip_uniforms(7, 0, 3, 81, 64))
    per = [(np.int32([1, 4, 9]), np.float32([2, 3, 4]), None), (np.int32([]), np.float32([]), None),
           (np.int32([4, 5]), np.float32([1.5, 8]), None)]
    blk, W = O.union_lists(per)
    np.testing.assert_array_equal(blk, [1, 4, 5, 9])
    np.testing.assert_array_equal(W, np.float32([[2, 0, 0], [3, 0, 1.5], [0, 0, 8], [4, 0, 0]]))


def test_cluster_estimator_all_blocks_is_dense_and_members_use_their_list():
    wl = gen_micro(4)
    B, H, L, d = wl.q.shape
    sigma = 1.0 / math.sqrt(d)
    per = O.select_clusters(wl.q, wl.k, wl.q_block, wl.kv_block, 1.0, C=2, mode=O.SEL_ALL)
    NQ = O.num_blocks(L, wl.q_block)
    for r_i, r in enumerate(per.rows):
        bh, i = divmod(r, NQ)
        b, h = divmod(bh, H)
        got = O.attend_row_clusters(wl.q, wl.k, wl.v, bh, i, wl.q_block, wl.kv_block, per.labels[r_i],
                                    per.lists[r_i], sigma)
        n = O.valid_len(i, wl.q_block, L)
        ref = O.dense_rows(wl.q, wl.k, wl.v, bh, i * wl.q_block, i * wl.q_block + n, sigma)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    # hand-made lists: a query of cluster 1 ignores cluster 0's list
    lab = np.zeros(wl.q_block, dtype=np.int64)
    lab[3] = 1
    lists = [(np.int32([0, 1]), np.float32([1, 1]), None), (np.int32([2]), np.float32([4]), None)]
    got = O.attend_row_clusters(wl.q, wl.k, wl.v, 0, 0, wl.q_block, wl.kv_block, lab, lists, sigma)
    num, den = O.estimator_num_den(wl.q[0, 0, [3]], wl.k[0, 0], wl.v[0, 0], [2], [4.0], wl.kv_block, sigma)
    np.testing.assert_allclose(got[3], (num / den[:, None])[0], rtol=1e-12)


def test_page_scale_budgets_sit_in_the_reported_skip_range():
    # The AB-Attention page reports 89-92% of the attention work skipped on Wan2.1 and
    # HunyuanVideo; the page-scale workloads keep the complementary 8-11% of the KV blocks.
    lo = 1.0 - page_figure("skipped_fraction_max")
    hi = 1.0 - page_figure("skipped_fraction_min")
    for cfg in (2, 3, 4):
        for keep in CONFIGS[cfg].keep:
            assert lo - 1e-9 <= keep <= hi + 1e-9, (cfg, keep)


# ----------------------------------------------------------------------------- second integer workload

def test_integer_family_guard_and_moving_kmeans_match_scipy():
    """The second integer workload (tests/exact_family.py): every block passes the fp32
    exactness guard; where the k-means still moves after its first step, the oracle's S2 equals
    scipy's kmeans2 step for step (it is the same Lloyd rule), and the guard rejects a block
    whose clustering mixes two families (a non-power-of-two normaliser)."""
    import warnings
    from exact_family import gen_exact_family
    from scipy.cluster.vq import kmeans2
    for C, Tk in ((2, 3), (4, 2), (8, 3)):
        wl = gen_exact_family(5, C, Tk)
        assert wl.extra["moved_blocks"] >= 8
        kbar = O.kv_block_means(wl.k[0, 0], 16)
        nk = np.full(64, 16.0)
        moved_seen = 0
        for i in range(16):
            X = wl.q[0, 0, i * 64:(i + 1) * 64].astype(np.float64)
            ok, moved = O.selection_fp32_exact(X, kbar, nk, C, Tk, 1.0, 16.0)
            assert ok
            mu, cnt, lab = O.ibcs_kmeans(X, C, Tk)
            init = np.stack([X[(j * 64) // C] for j in range(C)])
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                mu_s, lab_s = kmeans2(X, init, iter=Tk, minit="matrix", missing="warn")
            np.testing.assert_array_equal(mu, mu_s)
            np.testing.assert_array_equal(lab, lab_s)
            moved_seen += moved
        assert moved_seen >= 1
    # a block made of two families merged into one cluster is not exact
    from workloads import exact_family_block
    rng = np.random.default_rng(3)
    kbar = O.kv_block_means(gen_exact_family(1, 1, 1).k[0, 0], 16)
    rejected = 0
    for _ in range(40):
        X = exact_family_block(rng, families=2)
        ok, _ = O.selection_fp32_exact(X, kbar, np.full(64, 16.0), 1, 1, 1.0, 16.0)
        rejected += not ok
    assert rejected >= 30
