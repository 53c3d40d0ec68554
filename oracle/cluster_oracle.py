"""CPU oracle of per-cluster block lists (test infrastructure).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and the library never routes through it.

Sources: the PIVOT page (gyaansetu), section "PIVOT'un arkasındaki iki gözlem":
a proxy (the mean of a group of consecutive queries) is scored once and its
candidate list is then refined for each member of the group; the AB-Attention
page, section "AB-Attention ve Üç Temel Yeniliği", IBCS item: the proxies are
the centroids of the queries clustered inside each query block.  Here the
refinement is taken at cluster granularity: every cluster draws its own SIP
sample.  Readings (C1..C4), on top of S1..S6 of absa_oracle:

C1  Score of KV block b for cluster j: s_b^(j) = e_jb / Z_j, the centroid's
    own block distribution of S3 (sum over b is 1); the shared score of S3 is
    the mixture sum_j (n_j / n) s^(j).  A cluster with no member draws nothing
    (its list is empty in every mode).
C2  Each cluster gets the full budget n* = keep * NK and its own capped
    probabilities pi^(j) (S4) and Poisson draws (S5) with Philox counter word 1
    equal to i * C + j (so C = 1 reproduces the shared sample exactly).
C3  Query t of the block, in cluster a(t) (the last k-means assignment, S2),
    is estimated by S6 over cluster a(t)'s list with its weights.
C4  The lists of a row are handed to attention as their union in ascending
    block order with a weight per (entry, cluster), 0 where the cluster did
    not draw the block.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .absa_oracle import (SCORE_FLOOR_LOG2, SEL_ALL, SEL_SIP, SEL_TOPK, estimator_num_den, ibcs_kmeans,
                          kv_block_means, num_blocks, sip_inclusion, philox4x32_10, valid_len)

__all__ = ["cluster_scores", "cluster_uniforms", "select_row_cluster", "select_clusters", "ClusterSelect",
           "union_lists", "attend_row_clusters"]


def cluster_scores(mu: np.ndarray, counts: np.ndarray, kbar: np.ndarray, nk: np.ndarray,
                   alpha: float) -> np.ndarray:
    """C1: [C, NK] per-cluster block distributions (rows of empty clusters are 0)."""
    mu = np.asarray(mu, dtype=np.float64)
    kbar = np.asarray(kbar, dtype=np.float64)
    nk = np.asarray(nk, dtype=np.float64)
    C = mu.shape[0]
    s = np.zeros((C, kbar.shape[0]))
    for j in range(C):
        if counts[j] == 0:
            continue
        logit = alpha * (kbar @ mu[j])
        delta = logit - logit.max()
        e = np.where(delta >= SCORE_FLOOR_LOG2, nk * np.exp2(delta), 0.0)
        s[j] = e / e.sum()
    return s


def cluster_uniforms(seed: int, stream: int, bh: int, i: int, j: int, C: int, NK: int) -> np.ndarray:
    """C2: u_b of cluster j of row (bh, i): Philox counter (b // 4, i C + j, bh, stream)."""
    nctr = num_blocks(NK, 4)
    ctr = np.zeros((nctr, 4), dtype=np.uint32)
    ctr[:, 0] = np.arange(nctr, dtype=np.uint32)
    ctr[:, 1] = np.uint32((i * C + j) & 0xFFFFFFFF)
    ctr[:, 2] = np.uint32(bh)
    ctr[:, 3] = np.uint32(stream)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    x = philox4x32_10(ctr, key).reshape(-1)[:NK]
    return (x >> np.uint32(8)).astype(np.float64) * 2.0 ** -24


def select_row_cluster(s: np.ndarray, n_star: float, mode: int, u: np.ndarray, members: int = 1):
    """S4 + S5 (C2) for one cluster's scores: (kv_idx ascending, inv_pi fp32, pi_hat fp32)."""
    NK = s.shape[0]
    if members == 0:
        return np.zeros(0, np.int32), np.zeros(0, np.float32), np.zeros(NK, np.float32)
    if mode == SEL_ALL:
        return np.arange(NK, dtype=np.int32), np.ones(NK, dtype=np.float32), np.ones(NK, dtype=np.float32)
    if mode == SEL_TOPK:
        kstar = min(NK, int(math.floor(n_star + 0.5)))
        order = np.argsort(-s, kind="stable")
        kept = np.sort(order[:kstar]).astype(np.int32)
        pi_hat = np.zeros(NK, dtype=np.float32)
        pi_hat[kept] = 1.0
        return kept, np.ones(kept.shape[0], dtype=np.float32), pi_hat
    if mode != SEL_SIP:
        raise ValueError("unknown selection mode")
    pi_hat = sip_inclusion(s, n_star).astype(np.float32)
    kept = np.nonzero(u < pi_hat.astype(np.float64))[0].astype(np.int32)
    inv = (1.0 / pi_hat[kept].astype(np.float64)).astype(np.float32)
    return kept, inv, pi_hat


class ClusterSelect:
    """Per-row results: labels [n], and per cluster (kv_idx, inv_pi, pi_hat)."""

    def __init__(self):
        self.rows: List[int] = []
        self.labels: List[np.ndarray] = []
        self.lists: List[List[Tuple[np.ndarray, np.ndarray, np.ndarray]]] = []
        self.counts: List[np.ndarray] = []


def select_clusters(q: np.ndarray, k: np.ndarray, Bq: int, Bk: int, keep: float, C: int = 4, Tk: int = 3,
                    alpha: Optional[float] = None, sigma: Optional[float] = None, seed: int = 0,
                    stream: int = 0, mode: int = SEL_SIP, rows: Optional[Sequence[int]] = None) -> ClusterSelect:
    """S1, S2, C1, C2 over rows (bh, i) of q, k [B,H,L,d]."""
    B, H, L, d = q.shape
    NQ, NK = num_blocks(L, Bq), num_blocks(L, Bk)
    sigma = 1.0 / math.sqrt(d) if sigma is None or sigma <= 0 else sigma
    alpha = sigma * math.log2(math.e) if alpha is None or alpha <= 0 else alpha
    n_star = keep * NK
    rows = np.arange(B * H * NQ) if rows is None else np.asarray(rows, dtype=np.int64)
    nk = np.array([valid_len(b, Bk, L) for b in range(NK)], dtype=np.float64)
    kbar_cache: Dict[int, np.ndarray] = {}
    res = ClusterSelect()
    for r in rows:
        bh, i = divmod(int(r), NQ)
        b, h = divmod(bh, H)
        if bh not in kbar_cache:
            kbar_cache[bh] = kv_block_means(k[b, h], Bk)
        X = q[b, h, i * Bq: i * Bq + valid_len(i, Bq, L)]
        mu, cnt, lab = ibcs_kmeans(X, C, Tk)
        s = cluster_scores(mu, cnt, kbar_cache[bh], nk, alpha)
        per = []
        for j in range(C):
            u = cluster_uniforms(seed, stream, bh, i, j, C, NK)
            per.append(select_row_cluster(s[j], n_star, mode, u, int(cnt[j])))
        res.rows.append(int(r))
        res.labels.append(lab)
        res.lists.append(per)
        res.counts.append(cnt)
    return res


def union_lists(per: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """C4: (ascending union of the clusters' blocks, weights [n_union, C], 0 = not drawn)."""
    C = len(per)
    blocks = np.unique(np.concatenate([p[0] for p in per]).astype(np.int64)) if C else np.zeros(0, np.int64)
    W = np.zeros((blocks.shape[0], C), dtype=np.float32)
    pos = {int(b): n for n, b in enumerate(blocks)}
    for j, (idx, w, _) in enumerate(per):
        for b, wb in zip(idx, w):
            W[pos[int(b)], j] = wb
    return blocks.astype(np.int32), W


def attend_row_clusters(q, k, v, bh: int, i: int, Bq: int, Bk: int, labels: np.ndarray,
                        per: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]], sigma: float) -> np.ndarray:
    """C3: output [n_q(i), d] of row (bh, i), each query over its own cluster's list."""
    B, H, L, d = q.shape
    b, h = divmod(bh, H)
    n = valid_len(i, Bq, L)
    qb = np.asarray(q[b, h, i * Bq: i * Bq + n], dtype=np.float64)
    out = np.zeros((n, v.shape[-1]))
    for j, (idx, w, _) in enumerate(per):
        members = np.nonzero(labels[:n] == j)[0]
        if members.size == 0 or len(idx) == 0:
            continue
        num, den = estimator_num_den(qb[members], k[b, h], v[b, h], idx, w, Bk, sigma)
        nz = den > 0
        o = np.zeros_like(num)
        o[nz] = num[nz] / den[nz][:, None]
        out[members] = o
    return out
