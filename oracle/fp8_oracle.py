"""CPU oracle of the FP8 (e4m3) variant of the gather-attention step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and the library never routes through it.

Source: the VC-Attention page ("Nunchux AI'dan video difüzyon modellerini
hızlandıran VC-Attention", globalfeed), section "İki darboğaz": most of the
low-bit attention error comes from the value term; subtracting a per-block
mean of V before quantising removes part of the blocks' energy; the softmax
probabilities can be written as E4M3 bytes directly by one fused multiply-add,
because an E4M3 byte is close to a scaled log2 of the value it encodes
("ExpCast-FP8", mean deviation 1.6%); section "Ölçümler": such a kernel
composes with sparse attention.  The page names the ideas, not the formulas.
The readings used here:

F0  E4M3 is the OCP 8-bit format E4M3FN: bias 7, 3 mantissa bits, subnormals
    m 2^-9, largest finite 448, codes 0x7F / 0xFF are NaN, no infinities.
    Encoding rounds to nearest, ties to the even code; a negative input that
    rounds to zero gives -0 (0x80).  The scales below keep every quantised
    input within +-448 (beyond that the encoder here saturates).
    Every scale below is a power of two, s = 2^e with e the smallest integer
    for which max |x| <= 448 s (s = 1 for an all-zero set), so dividing by it
    is exact and only the E4M3 rounding loses information.
F1  Q: one scale per token, s_Q from max_c |q_c|, codes e4m3(q / s_Q).
F2  K: first centred by its per-head mean over all L tokens (a shift common to
    every key of a head leaves each query's softmax unchanged), k' = k - kbar
    in fp32; then one scale per KV block, s_K from max |k'| over the block's
    valid keys, codes e4m3(k' / s_K).
F3  V: per KV block the mean of its valid keys, rounded to bf16 (mu_hat); the
    residual r = v - mu_hat (fp32) is quantised with one scale per channel and
    head, s_V[c] from max_t |r[t][c]|, codes e4m3(r / s_V).  The value
    reconstructed for key t of block b is mu_hat_b + s_V * dec(code).
F4  Logits in log2 units: y = 8 (l - m) + 120 with l = sigma log2(e) s_Q s_K
    (q8 . k8) + log2 w_b, formed in fp32 by one fused multiply-add from the
    exact dot product of the codes: y = fp32(dot * M + c) with M = 8 fp32(sigma
    log2 e) s_Q s_K (exact: the scales are powers of two) and c = fp32(8
    fp32(fp32(log2 w) - m) + 120).  The reference m is one integer per query,
    fixed over the row's whole kept set: the smallest integer for which every
    kept key has y <= 120 (so the largest logit lands in (112, 120] and m =
    ceil(max l) up to the fp32 roundings of y).  It depends on the set of kept
    keys only, not on their order, and no running reference or rescaling
    enters the definition.
F5  ExpCast: p = dec_e4m3(sat_u8(rne(y))), the byte being y rounded to the
    nearest integer (ties to even) and clamped to [0, 255]; y <= 120 keeps it
    finite.  For bytes in the normal range 2^m dec(byte) does not depend on
    the integer m, so p is a fixed function of l (within 1.0615x of 2^l);
    bytes below 8 (y below 7.5) are E4M3 subnormals or zero, the underflow
    floor about 14 octaves below the largest term.
F6  o_t = sum_k p_k (mu_hat_b(k) + s_V dec(code_k)) / sum_k p_k over the row's
    kept keys (weights through log2 w inside l), the sums taken in ascending
    key order whatever the order of the list; an empty list gives 0.
F7  QK in INT8 instead (the page takes the QK side from earlier low-bit
    kernels such as SageAttention2, which smooth K and quantise QK to 8-bit
    integers): the same per-token Q and smoothed per-block K scaling with 127
    in place of 448 (s = 2^e, e smallest with max |x| <= 127 s), codes
    clip(rne(x / s), -127, 127); the dot products q8 . k8 are exact integers.

Every fp32 step that decides a code or a byte is taken in fp32 here as in the
kernel (numpy float32 arithmetic rounds each operation to nearest); the sums
that only accumulate are fp64.
"""
from __future__ import annotations

import math
from typing import NamedTuple, Optional, Sequence, Tuple

import numpy as np

from .absa_oracle import num_blocks, valid_len

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "bf16_round", "pow2_scale",
    "quantize_q", "smooth_k", "quantize_k", "quantize_v", "Fp8Head", "I8_MAX", "pow2_scale_i8", "i8_encode",
    "quantize_head", "expcast_p", "Fp8RowTerms", "fp8_row_terms", "attend_row_fp8", "attend_all_fp8",
]

E4M3_MAX = 448.0
I8_MAX = 127.0
EXPCAST_OFFSET = 120.0  # F4: the byte of the reference value 2^0 (a multiple of 8)

_F32 = np.float32


# ----------------------------------------------------------------------------- F0

def _decode_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * m * 2.0 ** -9
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_DEC = _decode_table()
_POS = _DEC[:127]  # finite non-negative values, increasing with the code


def e4m3_decode(codes) -> np.ndarray:
    """F0: value of each E4M3FN code (uint8 array) as fp64."""
    return _DEC[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """F0: round-to-nearest-even E4M3FN codes of fp32 values, saturating at +-448."""
    x = np.asarray(x, dtype=_F32).astype(np.float64)
    a = np.abs(x)
    lo = np.searchsorted(_POS, a, side="right") - 1          # largest code with value <= |x|
    lo = np.clip(lo, 0, 126)
    hi = np.minimum(lo + 1, 126)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    up = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    c = np.where(up & (lo < 126), hi, lo).astype(np.uint8)
    c = np.where(a >= E4M3_MAX, np.uint8(126), c)
    c = np.where(np.signbit(x), c | np.uint8(0x80), c)  # negative values rounding to 0 give -0
    c = np.where(np.isnan(x), np.uint8(0x7F), c)
    return c.astype(np.uint8)


def bf16_round(x) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    u = np.asarray(x, dtype=_F32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(_F32)


def pow2_scale(amax) -> np.ndarray:
    """2^e with e the smallest integer such that amax <= 448 * 2^e (1 where amax == 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, k = np.frexp(amax)                        # amax = m 2^k, m in [0.5, 1); 448 = 0.875 2^9
    e = np.where(m <= 0.875, k - 9, k - 8)
    return np.where(amax > 0, np.ldexp(1.0, e), 1.0).astype(_F32)


_scale = pow2_scale


def pow2_scale_i8(amax) -> np.ndarray:
    """F7: 2^e with e the smallest integer such that amax <= 127 * 2^e (1 where amax == 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, k = np.frexp(amax)                        # 127 = 0.9921875 2^7
    e = np.where(m <= 0.9921875, k - 7, k - 6)
    return np.where(amax > 0, np.ldexp(1.0, e), 1.0).astype(_F32)


def i8_encode(x) -> np.ndarray:
    """F7: clip(rne(x), -127, 127) as int8 codes (x already divided by its scale)."""
    x = np.asarray(x, dtype=_F32).astype(np.float64)
    return np.clip(np.rint(x), -127, 127).astype(np.int8)


# ----------------------------------------------------------------------------- F1-F3

def quantize_q(q: np.ndarray, int8: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """F1 (F7) for one head: q [L,d] (fp32 values of bf16) -> codes [L,d] (uint8 E4M3 or int8), s_Q [L]."""
    q = np.asarray(q, dtype=_F32)
    if int8:
        s = pow2_scale_i8(np.abs(q).max(axis=1))
        return i8_encode(q / s[:, None]), s
    s = _scale(np.abs(q).max(axis=1))
    return e4m3_encode(q / s[:, None]), s


def smooth_k(k: np.ndarray) -> np.ndarray:
    """F2: per-channel mean of all L keys of a head (fp64 sum, one rounding to fp32)."""
    k = np.asarray(k, dtype=np.float64)
    return (k.sum(axis=0) / k.shape[0]).astype(_F32)


def quantize_k(k: np.ndarray, Bk: int, int8: bool = False) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """F2 (F7) for one head: k [L,d] -> codes [L,d], s_K [NK] fp32, kbar [d] fp32."""
    L = k.shape[0]
    kbar = smooth_k(k)
    kc = np.asarray(k, dtype=_F32) - kbar[None, :]
    NK = num_blocks(L, Bk)
    s = np.empty(NK, dtype=_F32)
    codes = np.empty(kc.shape, dtype=np.int8 if int8 else np.uint8)
    for b in range(NK):
        t0, t1 = b * Bk, b * Bk + valid_len(b, Bk, L)
        amax = np.abs(kc[t0:t1]).max()
        s[b] = pow2_scale_i8(amax) if int8 else _scale(amax)
        codes[t0:t1] = i8_encode(kc[t0:t1] / s[b]) if int8 else e4m3_encode(kc[t0:t1] / s[b])
    return codes, s, kbar


def quantize_v(v: np.ndarray, Bk: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """F3 for one head: v [L,d] -> codes [L,d], s_V [d] fp32, mu_hat [NK,d] (bf16 values as fp32)."""
    L, d = v.shape
    NK = num_blocks(L, Bk)
    v32 = np.asarray(v, dtype=_F32)
    mu = np.empty((NK, d), dtype=_F32)
    for b in range(NK):
        t0, t1 = b * Bk, b * Bk + valid_len(b, Bk, L)
        mu[b] = (v32[t0:t1].astype(np.float64).sum(axis=0) / (t1 - t0)).astype(_F32)
    mu_hat = bf16_round(mu)
    r = v32 - np.repeat(mu_hat, Bk, axis=0)[:L]
    s = _scale(np.abs(r).max(axis=0))
    return e4m3_encode(r / s[None, :]), s, mu_hat


class Fp8Head:
    """F1-F3 (F7 for Q and K with ``qk_int8``) of one head: codes, scales and block means."""

    def __init__(self, q, k, v, Bk: int, qk_int8: bool = False):
        self.qk_int8 = bool(qk_int8)
        self.q8, self.sq = quantize_q(q, self.qk_int8)
        self.k8, self.sk, self.kbar = quantize_k(k, Bk, self.qk_int8)
        self.v8, self.sv, self.mu = quantize_v(v, Bk)
        self.Bk = Bk
        self.L = q.shape[0]

    def qk_values(self, codes) -> np.ndarray:
        """Values of Q or K codes (before their scales) as fp64."""
        return codes.astype(np.float64) if self.qk_int8 else e4m3_decode(codes)

    def values(self) -> np.ndarray:
        """Reconstructed V (F3) as fp64 [L, d]."""
        mu_k = np.repeat(self.mu.astype(np.float64), self.Bk, axis=0)[:self.L]
        return mu_k + e4m3_decode(self.v8) * self.sv.astype(np.float64)[None, :]


def quantize_head(q, k, v, Bk: int) -> Fp8Head:
    return Fp8Head(q, k, v, Bk)


# ----------------------------------------------------------------------------- F5

def expcast_p(y) -> np.ndarray:
    """F5: the probability written as the E4M3 byte sat_u8(rne(y)), as fp64."""
    y = np.asarray(y, dtype=np.float64)
    b = np.clip(np.rint(np.where(np.isnan(y), -1.0, y)), 0, 255).astype(np.int64)
    if np.any(b > 126):
        raise ValueError("ExpCast byte above the largest finite E4M3 code")
    return _DEC[b]


# ----------------------------------------------------------------------------- F4-F6

class Fp8RowTerms(NamedTuple):
    """The per-key terms of F4-F6 for a block of queries: keys in ascending order."""
    keys: np.ndarray     # [nk] int64 key indices
    dot: np.ndarray      # [n, nk] exact dot products q8 . k8 of the code values
    absdot: np.ndarray   # [n, nk] sum_i |q8_i k8_i| (the size of the dot product's terms)
    mul: np.ndarray      # [n, nk] M = 8 fp32(sigma log2 e) s_Q s_K
    add: np.ndarray      # [n, nk] c = fp32(8 fp32(fp32(log2 w) - m) + 120)
    m: np.ndarray        # [n] the integer reference of each query (F4)
    y: np.ndarray        # [n, nk] fp32 y
    p: np.ndarray        # [n, nk] F5 probabilities (fp64 values of E4M3 bytes)
    vals: np.ndarray     # [nk, d] reconstructed V (F3)
    mean: np.ndarray     # [nk, d] mu_hat of each key's block (the block-mean part of vals)


def _y_at(dot, mul, lw32, m) -> np.ndarray:
    """F4: fp32 y at integer references m [n] for all keys."""
    c = (lw32[None, :] - m.astype(_F32)[:, None]).astype(_F32)
    add = (c * _F32(8.0)).astype(np.float64) + EXPCAST_OFFSET
    add = add.astype(_F32).astype(np.float64)
    return (dot * mul + add).astype(_F32).astype(np.float64), add


def fp8_row_terms(hd: Fp8Head, t0: int, n: int, kept: Sequence[int], w: Sequence[float], sigma: float,
                  dense: bool = False) -> Optional[Fp8RowTerms]:
    """F4-F5 for queries t0 .. t0+n-1 of one head over the kept keys (every key with weight 1 if
    ``dense``); None for an empty list."""
    L, Bk = hd.L, hd.Bk
    if dense:
        blocks = np.arange(num_blocks(L, Bk), dtype=np.int64)
        wts = np.ones(blocks.size)
    else:
        if len(kept) == 0:
            return None
        order = np.argsort(np.asarray(kept, dtype=np.int64), kind="stable")   # the list is a set
        blocks = np.asarray(kept, dtype=np.int64)[order]
        wts = np.asarray(w, dtype=np.float64)[order]
    keys, lw = [], []
    for b, wb in zip(blocks, wts):
        nb = valid_len(int(b), Bk, L)
        keys.extend(range(int(b) * Bk, int(b) * Bk + nb))
        lw.extend([math.log2(float(wb))] * nb)
    keys = np.asarray(keys, dtype=np.int64)
    lw32 = np.asarray(lw, dtype=np.float64).astype(_F32)
    blk = keys // Bk
    sl2 = _F32(sigma * math.log2(math.e))
    qv = hd.qk_values(hd.q8[t0:t0 + n])
    kv = hd.qk_values(hd.k8[keys])
    dot = qv @ kv.T                                          # exact
    absdot = np.abs(qv) @ np.abs(kv).T
    mul = ((sl2 * hd.sq[t0:t0 + n]).astype(_F32)[:, None] * hd.sk[blk][None, :]).astype(_F32) * _F32(8.0)
    mul = mul.astype(np.float64)                             # exact products of powers of two and sl2
    # F4 reference: the smallest integer m with max_k y_k(m) <= 120; y(m) does not increase with m,
    # and ceil(max l) - 1 is below it (the fp32 roundings move y by far less than 8)
    lmax = (dot * mul / 8.0 + lw32[None, :]).max(axis=1)
    m = np.ceil(lmax) - 2.0
    for _ in range(6):
        y, _ = _y_at(dot, mul, lw32, m)
        over = y.max(axis=1) > EXPCAST_OFFSET
        if not over.any():
            break
        m = np.where(over, m + 1.0, m)
    y, add = _y_at(dot, mul, lw32, m)
    if (y.max(axis=1) > EXPCAST_OFFSET).any():
        raise AssertionError("F4 reference search did not settle")
    down, _ = _y_at(dot, mul, lw32, m - 1.0)
    if not (down.max(axis=1) > EXPCAST_OFFSET).all():
        raise AssertionError("F4 reference is not the smallest admissible integer")
    return Fp8RowTerms(keys=keys, dot=dot, absdot=absdot, mul=mul, add=add, m=m, y=y, p=expcast_p(y),
                       vals=hd.values()[keys], mean=hd.mu.astype(np.float64)[blk])


def attend_row_fp8(hd: Fp8Head, t0: int, n: int, kept: Sequence[int], w: Sequence[float],
                   sigma: float, dense: bool = False, expcast: bool = True) -> np.ndarray:
    """F4-F6 output [n, d] for queries t0 .. t0+n-1 of one head given its block list.

    With ``dense`` the list is ignored and every key is kept with weight 1.  ``expcast=False``
    replaces the F5 byte by the exact power 2^((y - 120) / 8) (used to check the rest of the
    assembly).
    """
    d = hd.q8.shape[1]
    t = fp8_row_terms(hd, t0, n, kept, w, sigma, dense)
    if t is None:
        return np.zeros((n, d))
    p = t.p if expcast else 2.0 ** ((t.y - EXPCAST_OFFSET) / 8.0)
    num = p @ t.vals
    den = p.sum(axis=1)
    out = np.zeros((n, d))
    nz = den > 0
    out[nz] = num[nz] / den[nz][:, None]
    return out


def attend_all_fp8(q, k, v, Bq: int, Bk: int, count=None, kv_idx=None, inv_pi=None,
                   sigma: Optional[float] = None, dense: bool = False,
                   rows: Optional[Sequence[int]] = None, qk_int8: bool = False) -> np.ndarray:
    """F1-F6 for the whole problem (or only ``rows``) -> O [B,H,L,d] fp64 (other rows zero)."""
    B, H, L, d = q.shape
    NQ = num_blocks(L, Bq)
    sigma = 1.0 / math.sqrt(d) if sigma is None or sigma <= 0 else sigma
    o = np.zeros((B, H, L, d))
    heads = {}
    rows = range(B * H * NQ) if rows is None else rows
    for r in rows:
        bh, i = divmod(int(r), NQ)
        b, h = divmod(bh, H)
        if bh not in heads:
            heads[bh] = Fp8Head(q[b, h], k[b, h], v[b, h], Bk, qk_int8)
        n = valid_len(i, Bq, L)
        if dense:
            o[b, h, i * Bq: i * Bq + n] = attend_row_fp8(heads[bh], i * Bq, n, [], [], sigma, dense=True)
        else:
            c = int(count[r])
            o[b, h, i * Bq: i * Bq + n] = attend_row_fp8(heads[bh], i * Bq, n, kv_idx[r, :c],
                                                         inv_pi[r, :c], sigma)
    return o
