"""Plain fp64 NumPy oracle of the AB-Attention hot path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and the library never routes through it.

Sources (the web pages this build works from):

* [AB] "AB-Attention: Video Difüzyon Transformer'larını Hızlandırmak İçin Doğru
  Blok Dikkat Mekanizması" (edumints blog).  Section "Video Difüzyon
  Modellerinde Dikkat Darboğazı" frames dynamic block-sparse attention and its
  three failure modes; section "AB-Attention ve Üç Temel Yeniliği" names IBCS
  (cluster the queries inside each query block, no token permutation), SIP
  (sample blocks in proportion to the IBCS estimates, reweight by the inverse
  inclusion probability, so one pass estimates dense attention) and the
  packed-tile kernel.
* [XA] "Cross-Attention (Çapraz Dikkat Mekanizması)" (yapayzekasozluk glossary),
  opening section and "Cross-Attention Nasıl Çalışır?": the formula
  softmax(Q K^T / sqrt(d_k)) V.
* [PV] the PIVOT page (gyaansetu), "PIVOT'un arkasındaki iki gözlem": a mean
  proxy of consecutive queries stands in for the group (the C = 1 case of the
  clustering below).

The pages fix none of IBCS/SIP's formulas.  The readings used here (each step
below says which) are:

S1  KV block summary = arithmetic mean of the block's valid keys.
S2  IBCS = Lloyd k-means on the raw query vectors of one query block, squared
    Euclidean distance, C clusters initialised at members floor(j n / C),
    Tk steps of (assign, update); ties go to the lowest cluster index; an empty
    cluster keeps its centroid.  Outputs the last centroids and the last counts.
S3  Score of KV block b = the estimated fraction of the query block's attention
    mass on b: a mixture over clusters (weight n_j / n) of each centroid's
    base-2 softmax over the block-mean logits alpha * mu_j . kbar_b, each term
    multiplied by the block's valid key count; terms with logit - max < -64 are 0.
S4  Inclusion probabilities pi_b = min(1, lambda s_b) with sum_b pi_b = n* =
    keep * NK, solved by iterative capping; pi is then rounded to fp32 and that
    fp32 value is used for the draw and for the weight.
S5  Poisson draws from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
    Random Numbers: As Easy as 1, 2, 3", SC'11): counter (floor(b/4), i, bh,
    stream), key (seed mod 2^32, seed div 2^32), word b mod 4, u = (x >> 8) 2^-24,
    keep b iff u < pi_hat_b; weight w_b = fp32(1 / pi_hat_b).
    TOPK: keep the k* = min(NK, floor(n* + 1/2)) largest scores (ties to the
    lower index), weight 1.  ALL: every block, weight 1.
S6  Estimator: o_t = sum_{b in S} w_b sum_{k in b} e^{a_k} v_k / sum_{b in S}
    w_b sum_{k in b} e^{a_k}, a_k = sigma q_t . k_k; the weights enter the
    softmax numerator and the denominator ([AB] SIP item).  Empty S gives 0.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "SEL_SIP", "SEL_TOPK", "SEL_ALL", "SCORE_FLOOR_LOG2",
    "num_blocks", "valid_len",
    "dense_attention", "dense_rows",
    "kv_block_means", "ibcs_kmeans", "ibcs_scores",
    "sip_inclusion", "bisection_inclusion",
    "philox4x32_10", "sip_uniforms",
    "select_row", "select", "SelectResult", "selection_fp32_exact",
    "estimator_num_den", "attend_row_block", "attend_rows", "attend_all", "sip_output_moments",
]

SEL_SIP, SEL_TOPK, SEL_ALL = 0, 1, 2
SCORE_FLOOR_LOG2 = -64.0  # S3: exp2 terms below this many octaves under the max are dropped


# ----------------------------------------------------------------------------- shapes

def num_blocks(L: int, block: int) -> int:
    """Number of blocks of ``block`` tokens covering L tokens (the last may be partial)."""
    return -(-L // block)


def valid_len(idx: int, block: int, L: int) -> int:
    """Valid tokens in block ``idx``: min(block, L - idx*block)."""
    return min(block, L - idx * block)


# ----------------------------------------------------------------------------- dense ([XA])

def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sigma: float) -> np.ndarray:
    """softmax(sigma Q K^T) V over all keys of one head ([XA] formula); q [n,d], k,v [L,d]."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    a = sigma * (q @ k.T)
    a -= a.max(axis=1, keepdims=True)
    p = np.exp(a)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def dense_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, bh: int, t0: int, t1: int,
               sigma: float) -> np.ndarray:
    """Dense attention output for queries [t0, t1) of flattened head bh; q,k,v [B,H,L,d]."""
    B, H, L, d = q.shape
    b, h = divmod(bh, H)
    return dense_attention(q[b, h, t0:t1], k[b, h], v[b, h], sigma)


# ----------------------------------------------------------------------------- S1

def kv_block_means(k: np.ndarray, Bk: int) -> np.ndarray:
    """S1: kbar_b = mean of the valid keys of KV block b; k [L,d] -> [NK,d] (fp64)."""
    k = np.asarray(k, dtype=np.float64)
    L = k.shape[0]
    NK = num_blocks(L, Bk)
    out = np.empty((NK, k.shape[1]), dtype=np.float64)
    for b in range(NK):
        out[b] = k[b * Bk: b * Bk + valid_len(b, Bk, L)].mean(axis=0)
    return out


# ----------------------------------------------------------------------------- S2 ([AB] IBCS)

def ibcs_kmeans(X: np.ndarray, C: int, Tk: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """S2: Lloyd k-means inside one query block (no reordering of the block's tokens).

    X [n,d] are the block's queries in token order.  Returns (mu [C,d], counts [C], labels [n])
    where counts/labels are those of the last assignment and mu the last update.
    """
    X = np.asarray(X, dtype=np.float64)
    n = X.shape[0]
    mu = np.stack([X[(j * n) // C] for j in range(C)])
    labels = np.zeros(n, dtype=np.int64)
    counts = np.zeros(C, dtype=np.int64)
    for _ in range(Tk):
        dist = ((X[:, None, :] - mu[None, :, :]) ** 2).sum(axis=2)  # [n, C]
        labels = np.argmin(dist, axis=1)  # first minimum = lowest cluster index
        counts = np.bincount(labels, minlength=C)
        new_mu = mu.copy()
        for j in range(C):
            if counts[j] > 0:
                new_mu[j] = X[labels == j].mean(axis=0)
        mu = new_mu
    return mu, counts, labels


# ----------------------------------------------------------------------------- S3 ([AB] IBCS)

def ibcs_scores(mu: np.ndarray, counts: np.ndarray, kbar: np.ndarray, nk: np.ndarray,
                alpha: float) -> np.ndarray:
    """S3: s_b = sum_j (n_j/n) * e_jb / Z_j with e_jb = nk_b * 2^(l_jb - m_j) (0 below the
    -64 floor), l_jb = alpha * mu_j . kbar_b, m_j = max_b l_jb, Z_j = sum_b e_jb.

    mu [C,d]; counts [C]; kbar [NK,d]; nk [NK] valid keys per block.  Sum of s is 1.
    """
    mu = np.asarray(mu, dtype=np.float64)
    kbar = np.asarray(kbar, dtype=np.float64)
    nk = np.asarray(nk, dtype=np.float64)
    n = float(np.sum(counts))
    s = np.zeros(kbar.shape[0], dtype=np.float64)
    for j in range(mu.shape[0]):
        if counts[j] == 0:
            continue
        logit = alpha * (kbar @ mu[j])
        delta = logit - logit.max()
        e = np.where(delta >= SCORE_FLOOR_LOG2, nk * np.exp2(delta), 0.0)
        s += (counts[j] / n) * e / e.sum()
    return s


# ----------------------------------------------------------------------------- S4 ([AB] SIP)

def sip_inclusion(s: np.ndarray, n_star: float) -> np.ndarray:
    """S4: capped inclusion probabilities pi_b = min(1, lambda s_b), sum pi = n* (fp64).

    Iterative capping: with U the uncapped positive blocks and R the budget left for them,
    every b in U with s_b * R >= sum_U s is set to 1 and removed, until none is; the rest get
    s_b * R / sum_U s.  n* >= NK gives pi = 1 everywhere; zero scores give pi = 0.
    """
    s = np.asarray(s, dtype=np.float64)
    NK = s.shape[0]
    if n_star >= NK:
        return np.ones(NK, dtype=np.float64)
    pi = np.zeros(NK, dtype=np.float64)
    U = s > 0
    R = float(n_star)
    while True:
        S_U = s[U].sum()
        N = U & (s * R >= S_U)
        if not N.any():
            break
        pi[N] = 1.0
        U &= ~N
        R -= int(N.sum())
        if not U.any():
            break
    if U.any():
        pi[U] = s[U] * R / s[U].sum()
    return pi


def bisection_inclusion(s: np.ndarray, n_star: float, iters: int = 200) -> np.ndarray:
    """Independent solver for the same pi: bisection on lambda in sum_b min(1, lambda s_b) = n*.

    (Used only to pin ``sip_inclusion``.)"""
    s = np.asarray(s, dtype=np.float64)
    pos = s > 0
    if n_star >= s.shape[0]:
        return np.ones_like(s)
    if n_star >= pos.sum():
        return pos.astype(np.float64)
    lo, hi = 0.0, 1.0 / s[pos].min()
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if np.minimum(1.0, mid * s).sum() < n_star:
            lo = mid
        else:
            hi = mid
    return np.minimum(1.0, 0.5 * (lo + hi) * s)


# ----------------------------------------------------------------------------- S5 Philox4x32-10

_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = np.uint32(0x9E3779B9)
_PHILOX_W1 = np.uint32(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """Philox4x32 with 10 rounds (SC'11 paper): ctr [...,4] uint32, key [...,2] uint32.

    One round multiplies words 0 and 2 by the two round multipliers into 64-bit products;
    the new block is (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)).
    The key is bumped by the two Weyl constants between rounds.
    """
    c = np.array(ctr, dtype=np.uint32, copy=True)
    k = np.broadcast_to(np.asarray(key, dtype=np.uint32), c.shape[:-1] + (2,)).copy()
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k[..., 0] += _PHILOX_W0
                k[..., 1] += _PHILOX_W1
            p0 = _PHILOX_M0 * c[..., 0].astype(np.uint64)
            p1 = _PHILOX_M1 * c[..., 2].astype(np.uint64)
            hi0 = (p0 >> np.uint64(32)).astype(np.uint32)
            lo0 = (p0 & _MASK32).astype(np.uint32)
            hi1 = (p1 >> np.uint64(32)).astype(np.uint32)
            lo1 = (p1 & _MASK32).astype(np.uint32)
            c = np.stack([hi1 ^ c[..., 1] ^ k[..., 0], lo1, hi0 ^ c[..., 3] ^ k[..., 1], lo0], axis=-1)
    return c


def sip_uniforms(seed: int, stream: int, bh: int, i: int, NK: int) -> np.ndarray:
    """S5: u_b for b < NK of row (bh, i): word b%4 of Philox(ctr=(b//4, i, bh, stream),
    key=(seed lo, seed hi)), u = (x >> 8) * 2^-24 (exact in fp32 and fp64)."""
    nctr = num_blocks(NK, 4)
    ctr = np.zeros((nctr, 4), dtype=np.uint32)
    ctr[:, 0] = np.arange(nctr, dtype=np.uint32)
    ctr[:, 1] = np.uint32(i)
    ctr[:, 2] = np.uint32(bh)
    ctr[:, 3] = np.uint32(stream)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    x = philox4x32_10(ctr, key).reshape(-1)[:NK]
    return (x >> np.uint32(8)).astype(np.float64) * 2.0 ** -24


# ----------------------------------------------------------------------------- selection driver

@dataclass
class SelectResult:
    count: np.ndarray          # [rows] int32
    kv_idx: List[np.ndarray]   # per row, ascending int32
    inv_pi: List[np.ndarray]   # per row, float32 weights
    pi_hat: np.ndarray         # [rows, NK] float32 (SIP: fp32 pi; TOPK: 1 kept / 0; ALL: 1)
    rows: np.ndarray           # flattened row ids bh*NQ + i that were computed
    scores: Optional[np.ndarray] = None   # [rows, NK] fp64
    mu: Optional[np.ndarray] = None       # [rows, C, d] fp64
    counts: Optional[np.ndarray] = None   # [rows, C]
    kbar: Optional[np.ndarray] = None     # [BH, NK, d] fp64


def select_row(s: np.ndarray, n_star: float, mode: int, seed: int, stream: int, bh: int,
               i: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """S4 + S5 for one row: returns (kv_idx int32 ascending, inv_pi float32, pi_hat float32)."""
    NK = s.shape[0]
    if mode == SEL_ALL:
        return (np.arange(NK, dtype=np.int32), np.ones(NK, dtype=np.float32),
                np.ones(NK, dtype=np.float32))
    if mode == SEL_TOPK:
        kstar = min(NK, int(math.floor(n_star + 0.5)))
        order = np.argsort(-s, kind="stable")  # descending; equal scores keep index order
        kept = np.sort(order[:kstar]).astype(np.int32)
        pi_hat = np.zeros(NK, dtype=np.float32)
        pi_hat[kept] = 1.0
        return kept, np.ones(kept.shape[0], dtype=np.float32), pi_hat
    if mode != SEL_SIP:
        raise ValueError("unknown selection mode")
    pi_hat = sip_inclusion(s, n_star).astype(np.float32)  # round to nearest fp32
    u = sip_uniforms(seed, stream, bh, i, NK)
    kept = np.nonzero(u < pi_hat.astype(np.float64))[0].astype(np.int32)
    inv = (1.0 / pi_hat[kept].astype(np.float64)).astype(np.float32)
    return kept, inv, pi_hat


def select(q: np.ndarray, k: np.ndarray, Bq: int, Bk: int, keep: float, C: int = 4, Tk: int = 3,
           alpha: Optional[float] = None, sigma: Optional[float] = None, seed: int = 0,
           stream: int = 0, mode: int = SEL_SIP, rows: Optional[Sequence[int]] = None,
           keep_intermediates: bool = False) -> SelectResult:
    """S1-S5 over the rows (bh, i) of q, k [B,H,L,d] (bf16 values widened to fp64).

    ``rows`` selects flattened row ids bh*NQ + i (default: all).  alpha defaults to
    sigma * log2(e) and sigma to 1/sqrt(d).
    """
    B, H, L, d = q.shape
    NQ, NK = num_blocks(L, Bq), num_blocks(L, Bk)
    sigma = 1.0 / math.sqrt(d) if sigma is None or sigma <= 0 else sigma
    alpha = sigma * math.log2(math.e) if alpha is None or alpha <= 0 else alpha
    n_star = keep * NK
    rows = np.arange(B * H * NQ) if rows is None else np.asarray(rows, dtype=np.int64)
    nk = np.array([valid_len(b, Bk, L) for b in range(NK)], dtype=np.float64)
    kbar_cache: Dict[int, np.ndarray] = {}
    counts_out = np.zeros(len(rows), dtype=np.int32)
    kv_idx, inv_pi = [], []
    pi_hat = np.zeros((len(rows), NK), dtype=np.float32)
    scores = np.zeros((len(rows), NK)) if keep_intermediates else None
    mus = np.zeros((len(rows), C, d)) if keep_intermediates else None
    cnts = np.zeros((len(rows), C), dtype=np.int64) if keep_intermediates else None
    for r_i, r in enumerate(rows):
        bh, i = divmod(int(r), NQ)
        b, h = divmod(bh, H)
        if bh not in kbar_cache:
            kbar_cache[bh] = kv_block_means(k[b, h], Bk)
        X = q[b, h, i * Bq: i * Bq + valid_len(i, Bq, L)]
        mu, cnt, _ = ibcs_kmeans(X, C, Tk)
        s = ibcs_scores(mu, cnt, kbar_cache[bh], nk, alpha)
        idx, w, ph = select_row(s, n_star, mode, seed, stream, bh, i)
        counts_out[r_i] = idx.shape[0]
        kv_idx.append(idx)
        inv_pi.append(w)
        pi_hat[r_i] = ph
        if keep_intermediates:
            scores[r_i], mus[r_i], cnts[r_i] = s, mu, cnt
    kbar = None
    if keep_intermediates:
        kbar = np.zeros((B * H, NK, d))
        for bh in range(B * H):
            b, h = divmod(bh, H)
            kbar[bh] = kbar_cache[bh] if bh in kbar_cache else kv_block_means(k[b, h], Bk)
    return SelectResult(count=counts_out, kv_idx=kv_idx, inv_pi=inv_pi, pi_hat=pi_hat, rows=rows,
                        scores=scores, mu=mus, counts=cnts, kbar=kbar)


# ----------------------------------------------------------------------------- exactness guard

def _f32_exact(x) -> bool:
    x = np.asarray(x, dtype=np.float64)
    return bool(np.all(x.astype(np.float32).astype(np.float64) == x))


def _split_bf16_exact(x) -> bool:
    """x equals bf16(x) + bf16(x - bf16(x)) (16 significant bits in two bf16 halves)."""
    x = np.asarray(x, dtype=np.float64).astype(np.float32)

    def bf(a):
        u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        return u.astype(np.uint32).view(np.float32)
    hi = bf(x)
    lo = bf((x - hi).astype(np.float32))
    return bool(np.all(hi.astype(np.float64) + lo.astype(np.float64) == x.astype(np.float64)))


def _granule(x: float) -> float:
    """The largest power of two dividing the positive float x."""
    m, e = math.frexp(x)                 # x = m 2^e, m in [0.5, 1)
    M = int(m * 2.0 ** 53)               # exact 53-bit integer
    tz = (M & -M).bit_length() - 1
    return math.ldexp(1.0, e - 53 + tz)


def _sums_exact(terms: np.ndarray) -> bool:
    """Every partial sum of the non-negative ``terms``, in any order, is exact in fp32: all are
    multiples of the smallest granule among them and the total stays below 2^24 of it."""
    t = np.asarray(terms, dtype=np.float64)
    t = t[t > 0]
    if t.size == 0:
        return True
    g = min(_granule(float(x)) for x in t)
    return bool(t.sum() < g * 2.0 ** 24)


def selection_fp32_exact(X: np.ndarray, kbar: np.ndarray, nk: np.ndarray, C: int, Tk: int, alpha: float,
                         n_star: float) -> Tuple[bool, bool]:
    """Exactness guard for the bit-exact selection tests (not a step of the method).

    Re-runs S2-S4 on one query block X [n,d] against the block means kbar [NK,d] and reports
    (exact, moved): ``exact`` when every intermediate a float32 implementation forms is exactly
    representable, so that float32 arithmetic in any summation order (with correctly rounded
    divisions and exact powers of two) reproduces the fp64 values and decisions of this oracle:
    the centroids of every step (also as two bf16 halves, the operands of a split-bf16 product),
    |mu|^2 and mu . x, every logit (an integer, so 2^(l - m) is exact), every term, normaliser and
    partial sum of S3, the mixture coefficients n_j / n / Z_j, every score, and every S_U and
    s_b R of the capping rounds.  ``moved``: the centroids still changed after the first step.
    """
    X = np.asarray(X, dtype=np.float64)
    n = X.shape[0]
    if not (_f32_exact(X) and _f32_exact(kbar) and _f32_exact(n_star)):
        return False, False
    mu = np.stack([X[(j * n) // C] for j in range(C)])
    counts = np.zeros(C, dtype=np.int64)
    moved = False
    for step in range(Tk):
        if not (_f32_exact(mu) and _split_bf16_exact(mu)):
            return False, moved
        sq = (mu * mu).sum(axis=1)
        G = X @ mu.T
        if not (_f32_exact(sq) and _f32_exact(G) and _f32_exact(sq[None, :] - 2.0 * G)):
            return False, moved
        dist = ((X[:, None, :] - mu[None, :, :]) ** 2).sum(axis=2)
        labels = np.argmin(dist, axis=1)
        counts = np.bincount(labels, minlength=C)
        new_mu = mu.copy()
        for j in range(C):
            if counts[j] > 0:
                tot = X[labels == j].sum(axis=0)
                if not _f32_exact(tot):
                    return False, moved
                new_mu[j] = tot / counts[j]
        if step >= 1 and not np.array_equal(new_mu, mu):
            moved = True
        mu = new_mu
    if not (_f32_exact(mu) and _split_bf16_exact(mu)):
        return False, moved
    s = np.zeros(kbar.shape[0])
    for j in range(C):
        if counts[j] == 0:
            continue
        logit = alpha * (np.asarray(kbar, dtype=np.float64) @ mu[j])
        if not (_f32_exact(logit) and np.all(logit == np.round(logit))):
            return False, moved
        delta = logit - logit.max()
        e = np.where(delta >= SCORE_FLOOR_LOG2, nk * np.exp2(delta), 0.0)
        Z = e.sum()
        coef = (counts[j] / n) / Z
        if not (_sums_exact(e) and _f32_exact(counts[j] / n) and _f32_exact(coef) and _f32_exact(coef * e)):
            return False, moved
        s += coef * e
        if not _f32_exact(s):
            return False, moved
    if not _sums_exact(s):
        return False, moved
    if n_star < s.shape[0]:
        U = s > 0
        R = float(n_star)
        while True:
            S_U = s[U].sum()
            if not (_f32_exact(S_U) and _f32_exact(s[U] * R) and _f32_exact(R)):
                return False, moved
            N = U & (s * R >= S_U)
            if not N.any():
                break
            U &= ~N
            R -= int(N.sum())
            if not U.any():
                break
    return True, moved


# ----------------------------------------------------------------------------- S6 ([AB] SIP)

def estimator_num_den(qb: np.ndarray, k: np.ndarray, v: np.ndarray, kept: Sequence[int],
                      w: Sequence[float], Bk: int, sigma: float,
                      shift: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """S6 numerator and denominator for the queries qb [n,d] of one query block.

    num_t = sum_{b in kept} w_b sum_{k in b} e^{a_tk - shift_t} v_k,
    den_t = sum_{b in kept} w_b sum_{k in b} e^{a_tk - shift_t},  a_tk = sigma q_t . k_k.
    ``shift`` defaults to the max of a over the kept keys (any common shift cancels in the ratio).
    """
    qb = np.asarray(qb, dtype=np.float64)
    L = k.shape[0]
    n, d = qb.shape
    if len(kept) == 0:
        return np.zeros((n, v.shape[1])), np.zeros(n)
    keys, wk = [], []
    for b, wb in zip(kept, w):
        t0, t1 = b * Bk, b * Bk + valid_len(int(b), Bk, L)
        keys.append(np.arange(t0, t1))
        wk.append(np.full(t1 - t0, float(wb)))
    keys = np.concatenate(keys)
    wk = np.concatenate(wk)
    a = sigma * (qb @ np.asarray(k[keys], dtype=np.float64).T)  # [n, nkeys]
    if shift is None:
        shift = a.max(axis=1)
    e = np.exp(a - shift[:, None]) * wk[None, :]
    num = e @ np.asarray(v[keys], dtype=np.float64)
    den = e.sum(axis=1)
    return num, den


def attend_row_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, bh: int, i: int, Bq: int,
                     Bk: int, kept: Sequence[int], w: Sequence[float], sigma: float) -> np.ndarray:
    """S6 output for the valid queries of row (bh, i) given its block list: [n_q(i), d]."""
    B, H, L, d = q.shape
    b, h = divmod(bh, H)
    qb = q[b, h, i * Bq: i * Bq + valid_len(i, Bq, L)]
    num, den = estimator_num_den(qb, k[b, h], v[b, h], kept, w, Bk, sigma)
    out = np.zeros_like(num)
    nz = den > 0
    out[nz] = num[nz] / den[nz][:, None]
    return out


def attend_rows(q, k, v, Bq: int, Bk: int, lists: Dict[int, Tuple[Sequence[int], Sequence[float]]],
                sigma: Optional[float] = None) -> Dict[int, np.ndarray]:
    """S6 for the rows in ``lists`` (row id -> (kv_idx, inv_pi)); returns row id -> [n_q, d]."""
    B, H, L, d = q.shape
    NQ = num_blocks(L, Bq)
    sigma = 1.0 / math.sqrt(d) if sigma is None or sigma <= 0 else sigma
    out = {}
    for r, (idx, w) in lists.items():
        bh, i = divmod(int(r), NQ)
        out[r] = attend_row_block(q, k, v, bh, i, Bq, Bk, idx, w, sigma)
    return out


def attend_all(q, k, v, Bq: int, Bk: int, count: np.ndarray, kv_idx: np.ndarray, inv_pi: np.ndarray,
               sigma: Optional[float] = None) -> np.ndarray:
    """S6 for every row from packed lists (count [rows], kv_idx/inv_pi [rows, cap]) -> O [B,H,L,d]."""
    B, H, L, d = q.shape
    NQ = num_blocks(L, Bq)
    sigma = 1.0 / math.sqrt(d) if sigma is None or sigma <= 0 else sigma
    o = np.zeros((B, H, L, d))
    for r in range(B * H * NQ):
        bh, i = divmod(r, NQ)
        b, h = divmod(bh, H)
        c = int(count[r])
        blk = attend_row_block(q, k, v, bh, i, Bq, Bk, kv_idx[r, :c], inv_pi[r, :c], sigma)
        o[b, h, i * Bq: i * Bq + blk.shape[0]] = blk
    return o


def sip_output_moments(qb: np.ndarray, k: np.ndarray, v: np.ndarray, pi_hat: np.ndarray, Bk: int,
                       sigma: float, max_free: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """First and second moments of the S6 output over the S5 Poisson draws of one row.

    pi_hat [NK] are the row's fp32 inclusion probabilities; block b is kept with probability
    pi_hat_b, independently, and then carries the weight fp32(1 / pi_hat_b) (S5).  Blocks with
    pi_hat 0 or 1 are fixed; the others (at most ``max_free``) are enumerated: every subset S
    has probability prod_{b in S} pi_b prod_{b not in S} (1 - pi_b), and o(S) is the S6 ratio
    (0 for an empty S).  Returns (E[o], E[o^2]) per element, [n, d] each.
    """
    qb = np.asarray(qb, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pi = np.asarray(pi_hat, dtype=np.float32).astype(np.float64)
    L, NK = k.shape[0], pi.shape[0]
    w = np.zeros(NK)
    w[pi > 0] = (1.0 / pi[pi > 0]).astype(np.float32).astype(np.float64)
    a = sigma * (qb @ k.T)                                  # [n, L]
    shift = a.max(axis=1, keepdims=True)
    e = np.exp(a - shift)
    n, d = qb.shape[0], v.shape[1]
    Nb = np.zeros((NK, n, d))
    Db = np.zeros((NK, n))
    for b in range(NK):
        t0, t1 = b * Bk, b * Bk + valid_len(b, Bk, L)
        Nb[b] = w[b] * (e[:, t0:t1] @ v[t0:t1])
        Db[b] = w[b] * e[:, t0:t1].sum(axis=1)
    fixed = np.flatnonzero(pi >= 1.0)
    free = np.flatnonzero((pi > 0.0) & (pi < 1.0))
    if free.size > max_free:
        raise ValueError("too many free blocks to enumerate")
    m1 = np.zeros((n, d))
    m2 = np.zeros((n, d))
    Nf = Nb[free].reshape(free.size, n * d)
    Df = Db[free]
    N0 = Nb[fixed].sum(axis=0).reshape(n * d)
    D0 = Db[fixed].sum(axis=0)
    total = 2 ** free.size
    for s0 in range(0, total, 2048):                         # subsets in chunks
        ids = np.arange(s0, min(total, s0 + 2048))
        masks = ((ids[:, None] >> np.arange(free.size)[None, :]) & 1).astype(np.float64)
        prob = np.prod(np.where(masks > 0, pi[free][None, :], 1.0 - pi[free][None, :]), axis=1)
        num = (N0[None] + masks @ Nf).reshape(-1, n, d)
        den = D0[None] + masks @ Df
        o = np.zeros_like(num)
        nz = den > 0
        o[nz] = num[nz] / den[nz][:, None]
        m1 += np.einsum("s,snd->nd", prob, o)
        m2 += np.einsum("s,snd->nd", prob, o * o)
    return m1, m2
