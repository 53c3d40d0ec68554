"""Pins of the FP8 oracle (F0..F6 in its header) against things other than itself: the
E4M3FN format's closed forms, torch's float8_e4m3fn conversion, the VC-Attention page's
ExpCast figure, the fp64 S6 estimator on inputs that quantise exactly, and invariances
the method must have."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from golden_figures import page_figure


# ----------------------------------------------------------------------------- F0

def test_e4m3_landmarks_and_order():
    dec = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert dec[0x00] == 0.0 and dec[0x01] == 2.0 ** -9 and dec[0x07] == 7 * 2.0 ** -9
    assert dec[0x08] == 2.0 ** -6 and dec[0x38] == 1.0 and dec[0x7E] == 448.0
    assert math.isnan(dec[0x7F]) and math.isnan(dec[0xFF])
    assert dec[0xB8] == -1.0 and dec[0xFE] == -448.0
    assert np.all(np.diff(dec[:127]) > 0)          # codes 0..126 increase
    np.testing.assert_array_equal(dec[0x80:0xFF], -dec[0x00:0x7F])


def test_e4m3_encode_matches_torch_float8():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(300000) * np.exp(rng.uniform(-14, 6.2, 300000))).astype(np.float32)
    x = x[np.abs(x) < 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(x), ref)


def test_e4m3_encode_ties_round_trip_and_sign():
    # every finite code round-trips; midpoints go to the even code
    codes = np.arange(127, dtype=np.uint8)
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_decode(codes).astype(np.float32)), codes)
    mids = ((O.e4m3_decode(codes[:-1]) + O.e4m3_decode(codes[1:])) / 2).astype(np.float32)
    got = O.e4m3_encode(mids)
    want = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    np.testing.assert_array_equal(got, want)
    assert O.e4m3_encode(np.float32(-1.0))[()] == 0xB8
    assert O.e4m3_encode(np.float32(-2.0 ** -11))[()] == 0x80  # rounds to -0


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)


def test_pow2_scale_is_the_smallest_power_of_two():
    rng = np.random.default_rng(7)
    a = (np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    a = np.concatenate([a, np.float32([448.0, 448.0 * 2 ** -5, 449.0, 224.0, 7.0, 1.0])])
    s = O.pow2_scale(a).astype(np.float64)
    assert np.all(a <= 448.0 * s) and np.all(a > 224.0 * s)
    assert O.pow2_scale(np.float32(448.0)) == 1.0 and O.pow2_scale(np.float32(449.0)) == 2.0
    assert O.pow2_scale(np.float32(0.0)) == 1.0


# ----------------------------------------------------------------------------- F5 (ExpCast)

def test_expcast_byte_reads_as_log2_within_closed_form_bound():
    # A normal byte B encodes (1 + f) 2^(e - 7) with B = 8 e + 8 f; read as 2^((B - 56)/8) the
    # ratio is (1 + f) / 2^f, between 1 and its maximum at f = 1/ln 2 - 1.
    B = np.arange(8, 127)
    ratio = O.e4m3_decode(B.astype(np.uint8)) / 2.0 ** ((B - 56) / 8.0)
    f = 1.0 / math.log(2.0) - 1.0
    rmax = (1.0 + f) / 2.0 ** f
    assert ratio.min() == 1.0 and ratio.max() <= rmax + 1e-15
    assert abs(rmax - 1.0615) < 1e-4


def test_expcast_mean_deviation_matches_page_figure():
    # The VC-Attention page puts the mean deviation of ExpCast at 1.6%.  The log-linear reading of
    # the byte (the approximation ExpCast rests on; scale constants cancel in the softmax) gives
    # a mean |deviation| from the exact power, around its mean ratio, of 1.53%.
    x = np.linspace(0.0, 8.0, 800001)[:-1]
    e = np.floor(x)
    f = x - e
    approx = (1.0 + f) * 2.0 ** e
    r = approx / 2.0 ** x
    dev = np.mean(np.abs(r / r.mean() - 1.0))
    assert abs(dev - page_figure("expcast_mean_abs_deviation")) < 0.001
    # and the oracle's byte rule realises that reading at integer bytes
    y = np.arange(8, 121, dtype=np.float64)
    np.testing.assert_array_equal(O.expcast_p(y), (1.0 + (y % 8) / 8.0) * 2.0 ** (np.floor(y / 8) - 7))


def test_expcast_shift_by_eight_doubles_and_floor():
    y = np.linspace(8.0, 112.0, 5001)
    np.testing.assert_array_equal(O.expcast_p(y + 8.0), 2.0 * O.expcast_p(y))
    assert O.expcast_p(np.array([-3.0, -0.4, np.nan]))[0] == 0.0
    assert O.expcast_p(np.array([-0.4]))[0] == 0.0 and O.expcast_p(np.array([0.6]))[0] == 2.0 ** -9
    with pytest.raises(ValueError):
        O.expcast_p(np.array([127.0]))


# ----------------------------------------------------------------------------- F1-F3

def test_quantisation_error_within_half_ulp():
    rng = np.random.default_rng(2)
    L, d, Bk = 100, 32, 16
    q = rng.standard_normal((L, d)).astype(np.float32)
    k = (rng.standard_normal((L, d)) + 3.0).astype(np.float32)
    v = (rng.standard_normal((L, d)) * np.exp(rng.uniform(-3, 3, (L, 1)))).astype(np.float32)
    hd = O.Fp8Head(q, k, v, Bk)

    def half_ulp(x):  # E4M3 spacing around |x|: 2^(e-3) for normals, 2^-9 below 2^-6
        ax = np.maximum(np.abs(x), 2.0 ** -6)
        return 2.0 ** (np.floor(np.log2(ax)) - 4)

    xq = q / hd.sq[:, None].astype(np.float64)
    assert np.all(np.abs(O.e4m3_decode(hd.q8) - xq) <= half_ulp(xq) * (1 + 1e-6))
    amax = np.abs(O.e4m3_decode(hd.q8)).max(axis=1)
    assert np.all((amax >= 224.0) & (amax <= 448.0))           # power-of-two scales use [224, 448]
    assert np.all(np.log2(hd.sq) == np.round(np.log2(hd.sq)))
    kc = k.astype(np.float64) - hd.kbar.astype(np.float64)
    np.testing.assert_allclose(hd.kbar, k.astype(np.float64).mean(axis=0), rtol=1e-6)
    for b in range(O.num_blocks(L, Bk)):
        sl = slice(b * Bk, min(L, (b + 1) * Bk))
        xk = kc[sl] / float(hd.sk[b])
        assert np.all(np.abs(O.e4m3_decode(hd.k8[sl]) - xk) <= half_ulp(xk) * (1 + 1e-5) + 1e-6)
        np.testing.assert_allclose(hd.mu[b], v[sl].astype(np.float64).mean(axis=0),
                                   rtol=2.0 ** -8, atol=1e-30)
    vr = hd.values()
    assert np.all(np.abs(vr - v) <= half_ulp((v - np.repeat(hd.mu, Bk, 0)[:L]) / hd.sv) * hd.sv * (1 + 1e-5)
                  + 1e-7)


# ----------------------------------------------------------------------------- F4-F6 assembly

def _exact_inputs(rng, L, d, Bk):
    """Q, K, V whose F1-F3 quantisation is exact: scales are 2^-6, K's mean is 0, every V block
    has a bf16 mean and a residual that sums to 0 within the block."""
    grid = O.e4m3_decode(np.arange(40, 126, dtype=np.uint8))      # magnitudes in [2^-2, 448)
    def pick(shape):
        return rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    q = pick((L, d)) * 2.0 ** -6
    q[:, 0] = 7.0                                                 # per-token max 448 * 2^-6
    half = L // 2
    kh = pick((half, d)) * 2.0 ** -6
    kh[:, 1] = 7.0
    k = np.concatenate([kh, -kh])                                 # exact zero mean
    NK = L // Bk
    mu = rng.integers(-8, 9, size=(NK, d)) / 4.0
    r = np.empty((L, d))
    for b in range(NK):
        rh = pick((Bk // 2, d)) * 2.0 ** -6
        rh = np.round(rh * 16) / 16                              # multiples of 1/16, still on the grid
        rh = np.where(rh == 0, 1.0 / 16, rh)
        rh[0, :] = 7.0
        r[b * Bk:(b + 1) * Bk] = np.concatenate([rh, -rh])
    v = np.repeat(mu, Bk, axis=0) + r
    for x in (q, k, v):   # all representable in bf16 and fp32
        assert np.array_equal(O.bf16_round(x.astype(np.float32)).astype(np.float64), x)
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


def test_assembly_equals_S6_estimator_on_exact_inputs():
    rng = np.random.default_rng(3)
    L, d, Bk = 256, 32, 16
    q, k, v = _exact_inputs(rng, L, d, Bk)
    hd = O.Fp8Head(q, k, v, Bk)
    np.testing.assert_array_equal(O.e4m3_decode(hd.q8) * hd.sq[:, None], q)
    np.testing.assert_array_equal(hd.values(), v)
    sigma = 0.05
    kept = [3, 0, 9, 15, 4, 7, 12]
    w = [1.5, 1.0, 3.25, 1.0, 8.0, 2.0, 1.125]
    got = O.attend_row_fp8(hd, 0, 64, kept, w, sigma, expcast=False)
    num, den = O.estimator_num_den(q[:64], k, v, kept, w, Bk, sigma)
    np.testing.assert_allclose(got, num / den[:, None], rtol=2e-5, atol=2e-5)


def test_list_order_does_not_change_the_output():
    # F4/F6: the reference is fixed over the row's whole kept set and the sums run in ascending key
    # order, so any permutation of a list (a set of blocks with their weights) gives the same bytes
    rng = np.random.default_rng(4)
    L, d, Bk = 512, 32, 16
    q = rng.standard_normal((L, d)).astype(np.float32)
    k = rng.standard_normal((L, d)).astype(np.float32)
    v = rng.standard_normal((L, d)).astype(np.float32)
    hd = O.Fp8Head(q, k, v, Bk)
    kept = list(range(0, 32, 1))
    w = list(2.0 ** rng.integers(0, 3, len(kept)) * rng.uniform(1.0, 1.5, len(kept)))
    a = O.attend_row_fp8(hd, 0, 40, kept, w, 0.2)
    for trial in range(3):
        perm = rng.permutation(len(kept))
        b = O.attend_row_fp8(hd, 0, 40, [kept[i] for i in perm], [w[i] for i in perm], 0.2)
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, O.attend_row_fp8(hd, 0, 40, kept[::-1], w[::-1], 0.2))


def test_reference_is_the_smallest_admissible_integer():
    # F4: per query, every y <= 120 and one octave down (m - 1) some y would exceed 120; the largest
    # term's byte therefore lies in [112, 120] and m = ceil(max l) wherever max l is not within the
    # fp32 roundings of an integer
    rng = np.random.default_rng(12)
    L, d, Bk = 384, 64, 16
    q = O.bf16_round(rng.standard_normal((L, d)).astype(np.float32) * 3)
    k = O.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    v = O.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    for qk_int8 in (False, True):
        hd = O.Fp8Head(q, k, v, Bk, qk_int8=qk_int8)
        kept = [1, 4, 5, 9, 17, 23]
        w = [1.0, 3.0, 1.25, 7.5, 2.0, 1.0]
        t = O.fp8_row_terms(hd, 64, 64, kept, w, 0.125)
        ymax = t.y.max(axis=1)
        assert np.all(ymax <= 120.0) and np.all(ymax >= 112.0 - 1e-3)
        l = t.dot * t.mul / 8.0 + np.log2(np.repeat(np.asarray(w), 16))[None, :]
        lmax = l.max(axis=1)
        clear = np.abs(lmax - np.round(lmax)) > 1e-3
        assert clear.sum() > 50
        np.testing.assert_array_equal(t.m[clear], np.ceil(lmax[clear]))
        # bytes of the largest terms: 112..120, the byte of 2^0 relative to the reference being 120
        assert np.all(np.rint(ymax) >= 112) and np.all(np.rint(ymax) <= 120)


def test_power_of_two_weights_shift_the_reference_only():
    # F4/F5: scaling every weight by 2^j shifts every l and the reference by j and leaves each y,
    # hence each byte and the output, unchanged; scaling one weight by 2 moves that block's bytes
    # up by exactly 8 (one E4M3 octave) where they stay normal
    rng = np.random.default_rng(13)
    L, d, Bk = 256, 32, 16
    q = rng.standard_normal((L, d)).astype(np.float32)
    k = rng.standard_normal((L, d)).astype(np.float32)
    v = rng.standard_normal((L, d)).astype(np.float32)
    hd = O.Fp8Head(q, k, v, Bk)
    kept = [0, 3, 6, 7, 11, 15]
    w = [1.0, 2.0, 4.0, 1.0, 8.0, 2.0]
    base = O.fp8_row_terms(hd, 0, 32, kept, w, 0.3)
    for j in (1, 5, 13):
        sh = O.fp8_row_terms(hd, 0, 32, kept, [x * 2.0 ** j for x in w], 0.3)
        np.testing.assert_array_equal(sh.m, base.m + j)
        np.testing.assert_array_equal(sh.y, base.y)
        np.testing.assert_array_equal(sh.p, base.p)
    w2 = list(w)
    w2[1] *= 2.0                                     # block 3 (keys 48..63 in ascending order)
    two = O.fp8_row_terms(hd, 0, 32, kept, w2, 0.3)
    same = two.m == base.m                          # queries whose largest term is elsewhere
    assert same.sum() >= 16
    cols = slice(16, 32)
    b0, b1 = np.rint(base.y[same][:, cols]), np.rint(two.y[same][:, cols])
    normal = b0 >= 8
    assert normal.sum() > 100
    np.testing.assert_array_equal(b1[normal], b0[normal] + 8)
    others = np.r_[0:16, 32:base.y.shape[1]]
    np.testing.assert_array_equal(two.y[same][:, others], base.y[same][:, others])


def test_key_shift_invariance_and_dense_equals_full_list():
    rng = np.random.default_rng(5)
    L, d, Bk = 320, 32, 16
    q = O.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    kh = rng.integers(-96, 97, size=(L // 2, d)) / 32.0
    k = np.concatenate([kh, -kh]).astype(np.float32)  # multiples of 1/32, mean exactly 0
    v = O.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    hd = O.Fp8Head(q, k, v, Bk)
    shift = np.float32(0.5) * np.sign(rng.standard_normal(d)).astype(np.float32)
    k2 = k + shift                                  # exact shift per channel, still bf16
    assert np.array_equal(O.bf16_round(k2), k2)
    assert np.array_equal(O.smooth_k(k2), shift)
    hd2 = O.Fp8Head(q, k2, v, Bk)
    np.testing.assert_array_equal(O.e4m3_decode(hd2.k8), O.e4m3_decode(hd.k8))  # (+0 and -0 alike)
    NK = L // Bk
    full = list(range(NK))
    a = O.attend_row_fp8(hd, 64, 64, full, [1.0] * NK, 0.1)
    b = O.attend_row_fp8(hd2, 64, 64, full, [1.0] * NK, 0.1)
    np.testing.assert_array_equal(a, b)
    c = O.attend_row_fp8(hd, 64, 64, [], [], 0.1, dense=True)
    np.testing.assert_array_equal(a, c)


def test_fp8_close_to_exact_attention_and_empty_list():
    rng = np.random.default_rng(6)
    L, d, Bk = 256, 64, 16
    q = O.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    k = O.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    v = O.bf16_round(rng.standard_normal((L, d)).astype(np.float32))
    hd = O.Fp8Head(q, k, v, Bk)
    sigma = 1.0 / math.sqrt(d)
    got = O.attend_row_fp8(hd, 0, 128, [], [], sigma, dense=True)
    ref = O.dense_attention(q[:128].astype(np.float64), k.astype(np.float64), v.astype(np.float64), sigma)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    # flat attention over 256 keys averages the values, so |o| ~ |v| / 16 while each term carries
    # ~2.6% (P) and ~3% (V) rounding: a relative error of a few percent is the expected size
    assert 0.005 < rel < 0.1
    assert np.all(O.attend_row_fp8(hd, 0, 16, [], [], sigma) == 0.0)


# ----------------------------------------------------------------------------- F7 (INT8 QK)

def test_i8_scale_rounding_and_error_bound():
    rng = np.random.default_rng(8)
    a = np.exp(rng.uniform(-20, 20, 20000)).astype(np.float32)
    s = O.pow2_scale_i8(a).astype(np.float64)
    assert np.all(a <= 127.0 * s) and np.all(a > 63.5 * s)
    assert O.pow2_scale_i8(np.float32(127.0)) == 1.0 and O.pow2_scale_i8(np.float32(127.5)) == 2.0
    # ties to even, clamping, exact integers
    np.testing.assert_array_equal(O.i8_encode(np.float32([0.5, 1.5, 2.5, -2.5, 126.5, 127.4, -300, 7])),
                                  np.int8([0, 2, 2, -2, 126, 127, -127, 7]))
    x = rng.standard_normal((64, 32)).astype(np.float32) * 5
    q8, sq = O.quantize_q(x, int8=True)
    err = np.abs(q8.astype(np.float64) * sq[:, None] - x)
    assert np.all(err <= sq[:, None] / 2 * (1 + 1e-7))
    assert np.all(np.abs(q8).max(axis=1) >= 63)


def test_int8_assembly_equals_S6_estimator_on_exact_inputs():
    rng = np.random.default_rng(9)
    L, d, Bk = 256, 32, 16
    q = rng.integers(-127, 128, size=(L, d)) * 2.0 ** -5
    q[:, 0] = 127 * 2.0 ** -5                                   # per-token max 127 * 2^-5
    kh = rng.integers(-127, 128, size=(L // 2, d)) * 2.0 ** -6
    kh[:, 1] = 127 * 2.0 ** -6
    k = np.concatenate([kh, -kh])                               # exact zero mean
    v = O.bf16_round(rng.standard_normal((L, d)).astype(np.float32)).astype(np.float64)
    q, k = q.astype(np.float32), k.astype(np.float32)
    hd = O.Fp8Head(q, k, v.astype(np.float32), Bk, qk_int8=True)
    np.testing.assert_array_equal(hd.q8.astype(np.float64) * hd.sq[:, None], q)
    for b in range(L // Bk):
        np.testing.assert_array_equal(hd.k8[b * Bk:(b + 1) * Bk].astype(np.float64) * hd.sk[b],
                                      k[b * Bk:(b + 1) * Bk])
    sigma = 0.05
    kept = [3, 0, 9, 15, 4, 7, 12]
    w = [1.5, 1.0, 3.25, 1.0, 8.0, 2.0, 1.125]
    got = O.attend_row_fp8(hd, 0, 64, kept, w, sigma, expcast=False)
    num, den = O.estimator_num_den(q[:64], k, hd.values(), kept, w, Bk, sigma)
    np.testing.assert_allclose(got, num / den[:, None], rtol=2e-5, atol=2e-5)
