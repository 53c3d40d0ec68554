"""CPU checks of the seeded input generators (`workloads/`) against their stated recipe: determinism,
head subsets, shapes and token grids, bf16-exact values, the outlier-token norm, and the structure of
the integer workload that makes its selection arithmetic exact."""
import numpy as np

from workloads import CONFIGS, bf16_round, gen_config, gen_exact, gen_fourier_heads, gen_micro


def test_same_seed_same_bytes_and_seeds_differ():
    a = gen_fourier_heads(2, 4, 5, 64, 4, 0.3, True, 11, [0, 1])
    b = gen_fourier_heads(2, 4, 5, 64, 4, 0.3, True, 11, [0, 1])
    c = gen_fourier_heads(2, 4, 5, 64, 4, 0.3, True, 12, [0, 1])
    for x, y, z in zip(a, b, c):
        assert x.tobytes() == y.tobytes()
        assert x.tobytes() != z.tobytes()


def test_head_subsets_keep_the_draws_of_the_full_workload():
    full = gen_config(1)
    sub = gen_config(1, heads=[1])
    for x, y in ((full.q, sub.q), (full.k, sub.k), (full.v, sub.v)):
        np.testing.assert_array_equal(x[:, 1:2], y)


def test_shapes_grids_and_bf16_values():
    for cfg, spec in CONFIGS.items():
        assert spec.T * spec.Hs * spec.Ws == spec.L
        wl = gen_config(cfg, heads=[0])
        assert wl.q.shape == (1, 1, spec.L, spec.d) and wl.L == spec.L
        assert (wl.T, wl.Hs, wl.Ws, wl.q_block, wl.kv_block) == (spec.T, spec.Hs, spec.Ws, spec.q_block,
                                                                spec.kv_block)
        for x in (wl.q, wl.k, wl.v):
            assert x.dtype == np.float32
            np.testing.assert_array_equal(bf16_round(x), x)   # every value is a bf16 value
    # the tiny workload keeps its fp32 originals for the oracle-only tests
    wl = gen_config(1)
    assert wl.q_f32 is not None and not np.array_equal(wl.q_f32, wl.q)


def test_outlier_tokens_have_ten_times_the_norm():
    T, Hs, Ws, d = 2, 10, 10, 64
    plain = gen_fourier_heads(T, Hs, Ws, d, 4, 0.3, False, 5, [0])
    out = gen_fourier_heads(T, Hs, Ws, d, 4, 0.3, True, 5, [0])
    for x0, x1 in zip(plain[:2], out[:2]):           # Q and K
        x0, x1 = x0[0].astype(np.float64), x1[0].astype(np.float64)
        changed = np.flatnonzero(np.any(x0 != x1, axis=1))
        assert len(changed) == int(np.ceil(0.005 * T * Hs * Ws))
        ratio = np.linalg.norm(x1[changed], axis=1) / np.linalg.norm(x0[changed], axis=1)
        np.testing.assert_allclose(ratio, 10.0, rtol=1e-5)
        # only four channels of each outlier token move
        assert all(int(np.sum(x0[p] != x1[p])) <= 4 for p in changed)
    np.testing.assert_array_equal(plain[2], out[2])  # V is untouched


def test_integer_workload_structure():
    for collapse in (False, True):
        wl = gen_exact(3, groups_collapse=collapse)
        L, d, Bk = wl.L, wl.d, wl.kv_block
        NK = L // Bk
        for h in range(wl.H):
            kb = wl.k[0, h].reshape(NK, Bk, d).astype(np.float64).mean(axis=1)
            np.testing.assert_array_equal(kb, np.eye(NK, d))   # block b's mean key is e_b
            q = wl.q[0, h].reshape(L // wl.q_block, 4, 16, d).astype(np.float64)
            centres = q.mean(axis=2)                           # zero-sum perturbations
            assert np.all(np.abs(wl.q[0, h]) <= 81) and np.all(wl.q[0, h] == np.round(wl.q[0, h]))
            for blk in centres:
                for c in blk:
                    a = c[c > -80.0]
                    s = np.sum(2.0 ** a)
                    assert s == 2.0 ** np.round(np.log2(s))         # the exponents sum to a power of two
                if collapse:
                    assert np.all(blk == blk[0])


def test_micro_workload_is_small_and_seeded():
    a, b, c = gen_micro(2), gen_micro(2), gen_micro(3)
    assert a.q.tobytes() == b.q.tobytes() and a.q.tobytes() != c.q.tobytes()
    assert a.q.shape == (1, 1, 256, 16) and a.L // a.kv_block == 16   # 2^16 Poisson subsets per row
