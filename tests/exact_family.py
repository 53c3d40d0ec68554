"""The second integer workload: query blocks whose selection stays exactly representable in
fp32 while the k-means moves (helpers, no tests).

Candidate blocks come from ``workloads.exact_family_block`` (groups of identical small-integer
rows, randomly interleaved, whose groups share active patterns by family); the oracle's
exactness guard keeps a candidate only if every intermediate of S2-S4 is exact in fp32 for the
given cluster count and step count.  With several steps, a share of the blocks is drawn among
candidates whose centroids still move after the first step, so the bit-exact comparison covers
k-means iterations that change the clustering."""
import numpy as np

import oracle as O
from workloads import Workload, bf16_round, exact_family_block, exact_keys

L, D, BQ, BK, NK = 1024, 64, 64, 16, 64
KEEP = 0.25


def gen_exact_family(seed: int, C: int, Tk: int, H: int = 2, moved_share: float = 0.5,
                     max_tries: int = 4000) -> Workload:
    """B=1, H heads, grid 4x16x16 (L=1024), d=64, Bq=64, Bk=16 (NK=64), keep 25%, alpha 1."""
    k = exact_keys(seed, H=H)
    q = np.zeros((1, H, L, D), dtype=np.float32)
    nk = np.full(NK, float(BK))
    rng = np.random.default_rng([seed, C, Tk, 9191])
    NQ = L // BQ
    n_moved = 0
    for h in range(H):
        kbar = O.kv_block_means(k[0, h], BK)
        for i in range(NQ):
            want_moved = Tk >= 2 and C >= 2 and (h * NQ + i) < moved_share * H * NQ
            for _ in range(max_tries):
                X = exact_family_block(rng, d=D, families=1 if C == 1 else None)
                exact, moved = O.selection_fp32_exact(X, kbar, nk, C, Tk, 1.0, KEEP * NK)
                if exact and (moved or not want_moved):
                    break
            else:
                raise RuntimeError(f"no exact candidate for C={C} Tk={Tk} block {h},{i}")
            n_moved += int(moved)
            q[0, h, i * BQ:(i + 1) * BQ] = X
    v = bf16_round(np.random.default_rng([seed, 9192]).standard_normal((1, H, L, D), dtype=np.float32))
    return Workload(q=q, k=k, v=v, B=1, H=H, L=L, d=D, T=4, Hs=16, Ws=16, q_block=BQ, kv_block=BK,
                    keep=KEEP, name=f"exact-integer family C={C} Tk={Tk}",
                    extra={"clusters": C, "kmeans_steps": Tk, "select_scale_log2": 1.0, "moved_blocks": n_moved})
