"""GPU parity of the FP8 (E4M3) path against the FP8 oracle (F0..F6 in oracle/fp8_oracle.py).

* Quantisation (absa_quantize_fp8): codes, scales, the key mean and the block-mean operands are
  bit-identical to the oracle's (every decision is an fp32 rounding both sides take in the same
  order; sums are exact fp64 sums of bf16 values).
* Attention (absa_attend_fp8): every output element lies within the element-wise bound of
  tests/fp8_bounds.py, derived from the kernel's arithmetic: the fp32 rounding of y (which can
  move a probability byte to its neighbour where y sits within that error of a rounding
  boundary), the underflow floor of the kernel's running reference (terms more than 14 octaves
  below a row's largest one), and the sums of the FP8 matrix instruction, which keeps its 64
  products to 13 bits below the largest one.  The whole output's rel-L2 must also stay within 3e-3.
  With INT8 QK the dot products are exact and every query gets a bound of its own; with E4M3 QK the
  instruction's alignment can move y by up to half a byte step on rows with outlier tokens, and
  queries whose bound would exceed their values' range are held to that range."""
import math
import sys

import numpy as np
import pytest

import oracle as O
from workloads import gen_config, gen_fourier_heads, bf16_round, Workload
from gpu_helpers import dev, lists_to_host, problem, sample_rows
from fp8_bounds import rows_reference_and_bound

pytestmark = pytest.mark.gpu

SIGMA128 = float(np.float32(1.0 / math.sqrt(128)))  # the scale the library derives for d = 128 (fp32)


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


def _workload(H, T, Hs, Ws, seed, outliers=False, modes=4):
    q, k, v = gen_fourier_heads(T, Hs, Ws, 128, modes, 0.3, outliers, seed, list(range(H)))
    L = T * Hs * Ws
    sh = (1, H, L, 128)
    return Workload(q=bf16_round(q.reshape(sh)), k=bf16_round(k.reshape(sh)), v=bf16_round(v.reshape(sh)),
                    B=1, H=H, L=L, d=128, T=T, Hs=Hs, Ws=Ws, q_block=128, kv_block=16, keep=0.25)


def _oracle_v8t(hd: O.Fp8Head) -> np.ndarray:
    L = hd.L
    NK = O.num_blocks(L, 16)
    v8 = np.zeros((NK * 16, 128), dtype=np.uint8)
    v8[:L] = hd.v8
    return v8.reshape(NK, 16, 128).transpose(0, 2, 1)          # [NK][c][key]


def _oracle_mu_op(hd: O.Fp8Head) -> np.ndarray:
    m = (hd.mu.astype(np.float64) / hd.sv.astype(np.float64)[None, :]).astype(np.float32)  # exact
    bits = (O.bf16_round(m).view(np.uint32) >> 16).astype(np.uint16)
    NK = bits.shape[0]
    return bits.reshape(NK, 4, 32).transpose(0, 2, 1)           # [NK][i][j] = channel 32 j + i


def _check_quantisation(ops, wl, heads):
    q8, sq, k8, sk = (t.cpu().numpy() for t in (ops.q8, ops.sq, ops.k8, ops.sk))
    if ops.qk_int8:
        q8, k8 = q8.view(np.int8), k8.view(np.int8)
    kbar, v8t, sv = ops.kbar.cpu().numpy(), ops.v8t.cpu().numpy(), ops.sv.cpu().numpy()
    mu = ops.mu.cpu().numpy().view(np.uint16)
    hds = {}
    for h in heads:
        hd = O.Fp8Head(wl.q[0, h], wl.k[0, h], wl.v[0, h], 16, qk_int8=ops.qk_int8)
        np.testing.assert_array_equal(q8[0, h], hd.q8, err_msg=f"Q codes head {h}")
        np.testing.assert_array_equal(sq[0, h], hd.sq, err_msg=f"s_Q head {h}")
        np.testing.assert_array_equal(kbar[0, h], hd.kbar, err_msg=f"kbar head {h}")
        np.testing.assert_array_equal(k8[0, h], hd.k8, err_msg=f"K codes head {h}")
        np.testing.assert_array_equal(sk[0, h], hd.sk, err_msg=f"s_K head {h}")
        np.testing.assert_array_equal(sv[0, h], hd.sv, err_msg=f"s_V head {h}")
        np.testing.assert_array_equal(v8t[0, h], _oracle_v8t(hd), err_msg=f"V codes head {h}")
        np.testing.assert_array_equal(mu[0, h], _oracle_mu_op(hd), err_msg=f"mean operands head {h}")
        hds[h] = hd
    return hds


def _compare(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str, int8_qk: bool = False, zones=0,
             ranged=0):
    """Every element within its derived bound (plus 1e-6 for the fp32 output itself) and the whole
    output's rel-L2 <= 3e-3.  With INT8 QK (exact dot products) every query has a bound of its
    own (none falls back to its values' range)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    slack = bound + 1e-6 + 2.0 ** -23 * np.abs(ref)
    worst = float((err / slack).max()) if err.size else 0.0
    _say(what, f"rel_l2={rel:.2e} max_abs={err.max():.2e} max err/bound={worst:.3f} "
               f"max bound={bound.max():.2e} median bound={np.median(bound):.2e} zone keys={zones} "
               f"queries bounded by range={ranged}")
    if int8_qk:
        assert ranged == 0, f"{what}: {ranged} queries without a bound of their own"
    bad = np.argwhere(err > slack)
    assert bad.size == 0, f"{what}: {len(bad)} elements beyond the bound, first {bad[:3].tolist()}, " \
                          f"err {err[tuple(bad[0])]:.3e} bound {slack[tuple(bad[0])]:.3e}"
    assert rel <= 3e-3, f"{what}: rel_l2={rel:.3e}"


def _oracle_rows(hds, wl, rows, count, kv_idx, inv_pi, NQ, dense=False, int8=False):
    return rows_reference_and_bound(hds, wl.L, rows, NQ, count, kv_idx, inv_pi, SIGMA128, int8, dense=dense)


def _check_rows(o, hds, wl, rows, count, kv_idx, inv_pi, NQ, what, int8=False, dense=False):
    refs, zones, ranged = _oracle_rows(hds, wl, rows, count, kv_idx, inv_pi, NQ, dense=dense, int8=int8)
    got = _gpu_rows(o, wl, rows, NQ)
    _compare(np.concatenate([got[r] for r in rows]), np.concatenate([refs[r][0] for r in rows]),
             np.concatenate([refs[r][1] for r in rows]), what, int8, zones, ranged)


def _gpu_rows(o, wl, rows, NQ):
    res = {}
    for r in rows:
        bh, i = divmod(int(r), NQ)
        res[int(r)] = o[0, bh, i * 128: min(wl.L, (i + 1) * 128)]
    return res


# ----------------------------------------------------------------------------- quantisation

@pytest.mark.parametrize("qk_int8", [False, True])
@pytest.mark.parametrize("shape", [
    dict(H=2, T=3, Hs=7, Ws=9),     # L = 189: ragged last KV block (13 keys) and query block
    dict(H=3, T=4, Hs=16, Ws=20),   # L = 1280
    dict(H=1, T=1, Hs=1, Ws=5),     # L = 5: one partial block
])
def test_quantize_bit_exact(absa, shape, qk_int8):
    wl = _workload(shape["H"], shape["T"], shape["Hs"], shape["Ws"], seed=21, outliers=True)
    p = problem(wl)
    ops, _ = absa.quantize_fp8(p, dev(wl.q), dev(wl.k), dev(wl.v), qk_int8=qk_int8)
    _check_quantisation(ops, wl, range(wl.H))


# ----------------------------------------------------------------------------- attention

def _random_lists(rng, rows, NK, keep, cap=None):
    cap = cap or NK
    count = np.zeros(rows, np.int32)
    idx = np.zeros((rows, cap), np.int32)
    w = np.ones((rows, cap), np.float32)
    for r in range(rows):
        sel = np.flatnonzero(rng.random(NK) < keep)
        count[r] = sel.size
        idx[r, :sel.size] = sel
        w[r, :sel.size] = (1.0 / rng.uniform(0.05, 1.0, sel.size)).astype(np.float32)
    return count, idx, w


def _to_lists(absa, count, idx, w):
    import torch
    return absa.BlockLists(torch.from_numpy(count).cuda(), torch.from_numpy(idx).cuda(),
                           torch.from_numpy(w).cuda())


@pytest.mark.parametrize("qk_int8", [False, True])
@pytest.mark.parametrize("shape,keep", [
    (dict(H=2, T=3, Hs=7, Ws=9), 0.5),       # L = 189
    (dict(H=2, T=4, Hs=16, Ws=20), 0.3),     # L = 1280
    (dict(H=1, T=5, Hs=19, Ws=23), 0.15),    # L = 2185, ragged
])
def test_attend_fp8_matches_oracle(absa, shape, keep, qk_int8):
    wl = _workload(shape["H"], shape["T"], shape["Hs"], shape["Ws"], seed=22)
    p = problem(wl)
    ops, _ = absa.quantize_fp8(p, dev(wl.q), dev(wl.k), dev(wl.v), qk_int8=qk_int8)
    hds = _check_quantisation(ops, wl, range(wl.H))
    rng = np.random.default_rng(5)
    count, idx, w = _random_lists(rng, p.rows, p.nk, keep)
    o = absa.attend_fp8(p, ops, _to_lists(absa, count, idx, w)).cpu().numpy()
    _check_rows(o, hds, wl, list(range(p.rows)), count, idx, w, p.nq,
                f"fp8 attend {shape} keep {keep} int8 QK {qk_int8}", qk_int8)


@pytest.mark.parametrize("qk_int8", [False, True])
@pytest.mark.parametrize("shape", [dict(H=2, T=3, Hs=7, Ws=9), dict(H=1, T=4, Hs=16, Ws=20)])
def test_dense_fp8_matches_oracle(absa, shape, qk_int8):
    wl = _workload(shape["H"], shape["T"], shape["Hs"], shape["Ws"], seed=23, outliers=True)
    p = problem(wl)
    ops, _ = absa.quantize_fp8(p, dev(wl.q), dev(wl.k), dev(wl.v), qk_int8=qk_int8)
    hds = _check_quantisation(ops, wl, range(wl.H))
    o = absa.attend_fp8(p, ops, None).cpu().numpy()
    _check_rows(o, hds, wl, list(range(p.rows)), None, None, None, p.nq, f"fp8 dense {shape} int8 QK {qk_int8}",
                qk_int8, dense=True)


def test_fp8_empty_invalid_and_bf16_output(absa):
    import torch
    wl = _workload(2, 2, 16, 20, seed=24)
    p = problem(wl)
    ops, _ = absa.quantize_fp8(p, dev(wl.q), dev(wl.k), dev(wl.v))
    hds = {h: O.Fp8Head(wl.q[0, h], wl.k[0, h], wl.v[0, h], 16) for h in range(wl.H)}
    rows, NK = p.rows, p.nk
    count = np.zeros(rows, np.int32)
    idx = np.zeros((rows, 8), np.int32)
    w = np.ones((rows, 8), np.float32)
    count[1] = 3
    idx[1, :3] = [2, NK + 5, 7]          # an index >= NK is skipped
    w[1, :3] = [2.0, 9.0, 1.5]
    count[2] = 99                        # clamped to cap = 8
    idx[2] = np.arange(0, 16, 2)
    o = absa.attend_fp8(p, ops, _to_lists(absa, count, idx, w)).cpu().numpy()
    assert np.all(o[0, 0, :128] == 0.0)  # empty list -> 0
    # the oracle sees what the kernel must use: entry NK + 5 skipped, the count clamped to cap = 8
    ec = np.array([0, 2, 8] + [0] * (rows - 3), np.int32)
    eidx = np.zeros((rows, 8), np.int32)
    ew = np.ones((rows, 8), np.float32)
    eidx[1, :2], ew[1, :2] = [2, 7], [2.0, 1.5]
    eidx[2] = np.arange(0, 16, 2)
    _check_rows(o, hds, wl, [1, 2], ec, eidx, ew, p.nq, "fp8 edge lists")
    pb = problem(wl, out_bf16=True)
    ob = absa.attend_fp8(pb, ops, _to_lists(absa, count, idx, w))
    assert ob.dtype == torch.bfloat16
    np.testing.assert_allclose(ob.float().cpu().numpy(), o, rtol=2 ** -8, atol=1e-6)


@pytest.mark.parametrize("qk_int8", [False, True])
def test_fp8_with_sip_lists_wan14b_720p(absa, qk_int8):
    """Full Wan2.1-14B 720p shape: quantisation of two heads bit-exact; attention on sampled rows
    (SIP lists from the library's own selection at keep 9.5%) against the oracle."""
    wl = _wan14b()
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    ops, _ = absa.quantize_fp8(p, q, k, v, qk_int8=qk_int8)
    hds = _check_quantisation(ops, wl, [0, wl.H - 1])
    lists, _, _ = absa.select(p, q, k, 0.095, seed=0)
    o = absa.attend_fp8(p, ops, lists).cpu().numpy()
    count, kv_idx, inv_pi = lists_to_host(lists)
    rng = np.random.default_rng(77)
    rows = [int(bh) * p.nq + int(i) for bh in hds for i in rng.choice(p.nq, 6, replace=False)]
    rows += [0, p.nq - 1, (wl.H - 1) * p.nq, wl.H * p.nq - 1]   # first and tail query blocks
    rows = sorted(set(rows))
    _check_rows(o, hds, wl, rows, count, kv_idx, inv_pi, p.nq,
                f"fp8 Wan14B 720p sampled rows ({len(rows)}) int8 QK {qk_int8}", qk_int8)


def test_fp8_maximum_kv_blocks(absa):
    """NK = 12288 (L = 196 608), the largest KV block count: quantisation bit-exact, attention on
    sampled rows with the library's SIP lists against the oracle."""
    wl = _workload(1, 48, 64, 64, seed=49, outliers=True)
    p = problem(wl)
    assert p.nk == 12288
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    ops, _ = absa.quantize_fp8(p, q, k, v)
    hds = _check_quantisation(ops, wl, [0])
    lists, _, _ = absa.select(p, q, k, 0.05, seed=3)
    o = absa.attend_fp8(p, ops, lists).cpu().numpy()
    count, kv_idx, inv_pi = lists_to_host(lists)
    rng = np.random.default_rng(78)
    rows = sorted(set(int(i) for i in rng.choice(p.nq, 8, replace=False)) | {0, p.nq - 1})
    _check_rows(o, hds, wl, rows, count, kv_idx, inv_pi, p.nq, f"fp8 NK = 12288 sampled rows ({len(rows)})")


@pytest.mark.parametrize("qk_int8", [False, True])
def test_fp8_deterministic(absa, qk_int8):
    """Two runs of quantisation and attention give the same bytes (no order-dependent sums)."""
    import torch
    wl = _workload(2, 5, 15, 16, seed=31, outliers=True)
    p = problem(wl)
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists, _, _ = absa.select(p, q, k, 0.2, seed=4)
    outs = []
    for _ in range(2):
        ops, _ = absa.quantize_fp8(p, q, k, v, qk_int8=qk_int8)
        o = absa.attend_fp8(p, ops, lists)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (ops.q8, ops.sq, ops.k8, ops.sk, ops.kbar, ops.v8t, ops.sv, ops.mu, o)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


_WAN14 = {}


def _wan14b():
    if "wl" not in _WAN14:
        _WAN14["wl"] = gen_config(3)
    return _WAN14["wl"]
