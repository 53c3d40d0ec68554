"""Seeded synthetic Q/K/V generators for video-DiT-shaped attention workloads.

The AB-Attention page (edumints blog, section "Performans Sonuçları ve Pratik
Çıkarımlar") measures on Wan2.1 and HunyuanVideo generation; the VC-Attention
page (globalfeed, opening section) describes a clip flattened to one
spatiotemporal token sequence (a 5 s 720p clip is about 70 K tokens).  Neither
trained weights nor prompts exist here, so these generators stand in for the
models' attention inputs with their head count, head dimension and token grid.

Recipe (every draw comes from ``numpy.random.default_rng`` seeded by
``(data_seed, head, stream)``, so any subset of heads can be regenerated alone):

* token order is raster over the (T, Hs, Ws) grid, t-major, x fastest;
* per head, M modes with integer frequencies f_a ~ U{0..min(3, n_a // 2)} per
  axis and phase phi ~ U[0, 2 pi); Q and K share the modes (one field per
  head) and draw independent amplitudes A_Q, A_K ~ N(0, 1) of shape [M, d];
* X(t, y, x) = sum_m A_X[m] cos(2 pi (f_t t/T + f_y y/Hs + f_x x/Ws) + phi_m)
  plus N(0, noise_std) noise (``noise_std`` is a standard deviation);
* optional outliers: ceil(0.005 L) token positions per head, the same in Q and
  K; at each, 4 random channels (shared by Q and K) are overwritten with
  independent +-a so that the token's norm becomes exactly 10x its old norm;
* V ~ N(0, 1);
* values are rounded to bf16 with round-to-nearest-even and returned as
  float32 arrays holding bf16-exact values (``bf16_bits`` gives the raw bits).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "CONFIGS",
    "Workload",
    "bf16_round",
    "bf16_bits",
    "gen_config",
    "gen_exact",
    "exact_keys",
    "exact_family_block",
    "gen_micro",
    "gen_fourier_heads",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of an array that is already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array holds values that are not bf16-exact")
    return (u >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    name: str
    B: int
    H: int
    d: int
    T: int
    Hs: int
    Ws: int
    modes: int
    noise_std: float
    outliers: bool
    q_block: int
    kv_block: int
    keep: Sequence[float]

    @property
    def L(self) -> int:
        return self.T * self.Hs * self.Ws


# The workloads, named by the model shape they imitate.
CONFIGS: Dict[int, ConfigSpec] = {
    1: ConfigSpec("tiny 4x16x16", 1, 2, 64, 4, 16, 16, 4, 0.3, False, 64, 16, (0.25,)),
    2: ConfigSpec("Wan2.1-1.3B-shaped 480p", 1, 12, 128, 21, 30, 52, 16, 0.5, True, 64, 16, (0.10,)),
    3: ConfigSpec("Wan2.1-14B-shaped 720p", 1, 40, 128, 21, 45, 80, 32, 0.5, True, 128, 16,
                  (0.08, 0.095, 0.11)),
    4: ConfigSpec("HunyuanVideo-shaped 720p", 1, 24, 128, 33, 45, 80, 32, 0.5, True, 128, 16, (0.08,)),
}


@dataclasses.dataclass
class Workload:
    """Q, K, V as float32 arrays [B, H, L, d] holding bf16-exact values."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    B: int
    H: int
    L: int
    d: int
    T: int
    Hs: int
    Ws: int
    q_block: int
    kv_block: int
    keep: float
    name: str = ""
    q_f32: Optional[np.ndarray] = None  # unrounded values where the workload is fp32
    k_f32: Optional[np.ndarray] = None
    v_f32: Optional[np.ndarray] = None
    extra: Optional[dict] = None


def _grid_phase(T: int, Hs: int, Ws: int, freqs: np.ndarray, phases: np.ndarray) -> np.ndarray:
    """cos(2 pi (f . coords / grid) + phi) for every token (raster order) and mode: [L, M]."""
    t = np.arange(T, dtype=np.float64)[:, None, None] / T
    y = np.arange(Hs, dtype=np.float64)[None, :, None] / Hs
    x = np.arange(Ws, dtype=np.float64)[None, None, :] / Ws
    cols = []
    for m in range(freqs.shape[0]):
        ft, fy, fx = freqs[m]
        ang = 2.0 * np.pi * (ft * t + fy * y + fx * x) + phases[m]
        cols.append(np.cos(ang).reshape(-1))
    return np.stack(cols, axis=1)


def _one_head(spec_like, data_seed: int, h: int):
    T, Hs, Ws, d, M = spec_like["T"], spec_like["Hs"], spec_like["Ws"], spec_like["d"], spec_like["modes"]
    L = T * Hs * Ws
    rng = np.random.default_rng([data_seed, h, 0])
    fmax = np.array([min(3, T // 2), min(3, Hs // 2), min(3, Ws // 2)])
    freqs = np.stack([rng.integers(0, fmax[a] + 1, size=M) for a in range(3)], axis=1)
    phases = rng.uniform(0.0, 2.0 * np.pi, size=M)
    basis = _grid_phase(T, Hs, Ws, freqs, phases).astype(np.float32)  # [L, M]
    a_q = rng.standard_normal((M, d), dtype=np.float32)
    a_k = rng.standard_normal((M, d), dtype=np.float32)
    q = basis @ a_q
    k = basis @ a_k
    rng_n = np.random.default_rng([data_seed, h, 1])
    q += rng_n.standard_normal((L, d), dtype=np.float32) * np.float32(spec_like["noise_std"])
    k += rng_n.standard_normal((L, d), dtype=np.float32) * np.float32(spec_like["noise_std"])
    if spec_like["outliers"]:
        rng_o = np.random.default_rng([data_seed, h, 3])
        n_out = int(math.ceil(0.005 * L))
        pos = rng_o.choice(L, size=n_out, replace=False)
        for p in pos:
            ch = rng_o.choice(d, size=4, replace=False)
            for x in (q, k):
                row = x[p].astype(np.float64)
                norm2 = float(row @ row)
                rest = row.copy()
                rest[ch] = 0.0
                rest2 = float(rest @ rest)
                a = math.sqrt(max(100.0 * norm2 - rest2, 0.0) / 4.0)
                signs = rng_o.choice(np.array([-1.0, 1.0]), size=4)
                row[ch] = signs * a
                x[p] = row.astype(np.float32)
    rng_v = np.random.default_rng([data_seed, h, 2])
    v = rng_v.standard_normal((L, d), dtype=np.float32)
    return q, k, v


def gen_fourier_heads(T: int, Hs: int, Ws: int, d: int, modes: int, noise_std: float, outliers: bool,
                      data_seed: int, heads: Sequence[int], round_bf16: bool = False):
    """Float32 Q, K, V of shape [len(heads), L, d] for the given head indices (rounded to
    bf16 values when ``round_bf16``)."""
    spec_like = dict(T=T, Hs=Hs, Ws=Ws, d=d, modes=modes, noise_std=noise_std, outliers=outliers)
    L = T * Hs * Ws
    out = [np.empty((len(heads), L, d), dtype=np.float32) for _ in range(3)]

    def fill(n_h):
        n, h = n_h
        q, k, v = _one_head(spec_like, data_seed, h)
        if round_bf16:
            q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
        out[0][n], out[1][n], out[2][n] = q, k, v

    # Heads are independent draws; threads only overlap numpy's GIL-free work.
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, max(1, len(heads)))) as ex:
        list(ex.map(fill, enumerate(heads)))
    return out


def gen_config(cfg: int, heads: Optional[Sequence[int]] = None, keep: Optional[float] = None,
               kv_block: Optional[int] = None, data_seed: Optional[int] = None) -> Workload:
    """Generate workload ``cfg`` (1..4).  ``heads`` restricts H to a subset of head indices
    (they keep the draws of the full workload); ``data_seed`` defaults to the workload id."""
    spec = CONFIGS[cfg]
    heads = list(range(spec.H)) if heads is None else list(heads)
    seed = cfg if data_seed is None else data_seed
    keep_raw = cfg == 1
    q, k, v = gen_fourier_heads(spec.T, spec.Hs, spec.Ws, spec.d, spec.modes, spec.noise_std,
                                spec.outliers, seed, heads, round_bf16=not keep_raw)
    shape = (1, len(heads), spec.L, spec.d)
    q, k, v = q.reshape(shape), k.reshape(shape), v.reshape(shape)
    qr, kr, vr = (bf16_round(q), bf16_round(k), bf16_round(v)) if keep_raw else (q, k, v)
    wl = Workload(q=qr, k=kr, v=vr, B=1, H=len(heads), L=spec.L,
                  d=spec.d, T=spec.T, Hs=spec.Hs, Ws=spec.Ws, q_block=spec.q_block,
                  kv_block=spec.kv_block if kv_block is None else kv_block,
                  keep=spec.keep[0] if keep is None else keep, name=spec.name)
    if keep_raw:
        wl.q_f32, wl.k_f32, wl.v_f32 = q, k, v
    return wl


def gen_micro(data_seed: int = 1) -> Workload:
    """Tiny shape for exhaustive enumeration of Poisson subsets: B=H=1, d=16, grid 1x16x16
    (L=256), query block 64, KV block 16 (16 KV blocks), keep 25%; data from the tiny
    workload's recipe (4 modes, noise std 0.3)."""
    q, k, v = gen_fourier_heads(1, 16, 16, 16, 4, 0.3, False, data_seed, [0])
    shape = (1, 1, 256, 16)
    return Workload(q=bf16_round(q.reshape(shape)), k=bf16_round(k.reshape(shape)),
                    v=bf16_round(v.reshape(shape)), B=1, H=1, L=256, d=16, T=1, Hs=16, Ws=16,
                    q_block=64, kv_block=16, keep=0.25, name="micro")


def gen_exact(seed: int = 0, H: int = 2, groups_collapse: bool = False) -> Workload:
    """Small-integer Q/K whose selection arithmetic is exact in fp32.

    Shape: B=1, H heads, d=64, grid 4x16x16 (L=1024), query block 64, KV block 16 (so the
    number of KV blocks equals d = 64), keep 25%.  Intended with 4 clusters, 3 k-means steps
    and selection logit scale 1.

    Keys: KV block b holds e_b (one-hot at channel b) plus integer perturbations in {-1,0,1}
    that sum to zero over the block's 16 keys, so its mean key is exactly e_b.

    Queries: query block i is 4 contiguous groups of 16 rows; group j is a centre a_ij plus
    zero-sum {-1,0,1} perturbations.  Centres differ by >= 70 in some channel, so evenly
    spaced initial centroids land one per group and every k-means step recovers the centres
    exactly.  Centre j puts an exponent multiset on a random set of channels (= KV blocks):
    it starts from {E} (E ~ U{0..6}) and repeatedly splits a term e into two terms e-1 (depth
    <= 10), so sum_b 2^a_ij[b] is a power of two; all other channels hold -80.  Values are
    integers with |x| <= 81, exact in bf16.

    ``groups_collapse``: every row of a query block equals one centre (no perturbation): all
    distances tie, so every query joins cluster 0 (lowest-index rule) and clusters 1..3 stay
    empty with their initial centroids.
    """
    B, d, T, Hs, Ws = 1, 64, 4, 16, 16
    L = T * Hs * Ws
    Bq, Bk = 64, 16
    NQ, NK = L // Bq, L // Bk
    rng = np.random.default_rng([seed, 7777])
    q = np.zeros((B, H, L, d), dtype=np.float32)
    k = np.zeros((B, H, L, d), dtype=np.float32)

    def zero_sum_perturb(rows: int) -> np.ndarray:
        p = np.zeros((rows, d), dtype=np.float32)
        for c in range(d):
            j = int(rng.integers(0, rows // 2 + 1))
            idx = rng.permutation(rows)[: 2 * j]
            p[idx[:j], c] = 1.0
            p[idx[j:], c] = -1.0
        return p

    for h in range(H):
        for b in range(NK):
            blk = zero_sum_perturb(Bk)
            blk[:, b] += 1.0
            k[0, h, b * Bk:(b + 1) * Bk] = blk
        for i in range(NQ):
            centres = []
            while len(centres) < 4:
                j = len(centres)
                if groups_collapse and j > 0:
                    centres.append(centres[0].copy())
                    continue
                E = int(rng.integers(0, 7))
                terms = [E]
                n_split = int(rng.integers(0, 16))
                for _ in range(n_split):
                    cand = [t for t in range(len(terms)) if terms[t] > E - 10]
                    if not cand:
                        break
                    t = cand[int(rng.integers(0, len(cand)))]
                    e = terms.pop(t)
                    terms += [e - 1, e - 1]
                chans = rng.choice(d, size=len(terms), replace=False)
                a = np.full(d, -80.0, dtype=np.float32)
                a[chans] = np.asarray(terms, dtype=np.float32)
                if all(np.max(np.abs(a - c)) >= 70.0 for c in centres):
                    centres.append(a)
            rows = np.zeros((Bq, d), dtype=np.float32)
            for j in range(4):
                pert = np.zeros((16, d), np.float32) if groups_collapse else zero_sum_perturb(16)
                rows[16 * j:16 * (j + 1)] = centres[j][None, :] + pert
            q[0, h, i * Bq:(i + 1) * Bq] = rows
    v = bf16_round(np.random.default_rng([seed, 7778]).standard_normal((B, H, L, d), dtype=np.float32))
    return Workload(q=q, k=k, v=v, B=B, H=H, L=L, d=d, T=T, Hs=Hs, Ws=Ws, q_block=Bq, kv_block=Bk,
                    keep=0.25, name="exact-integer", extra={"clusters": 4, "kmeans_steps": 3,
                                                           "select_scale_log2": 1.0})


def exact_keys(seed: int, H: int = 2, L: int = 1024, d: int = 64, Bk: int = 16) -> np.ndarray:
    """Keys [1, H, L, d] whose KV block b (Bk keys) is e_b (one-hot at channel b) plus integer
    perturbations in {-1, 0, 1} that sum to zero over the block, so its mean key is exactly e_b
    (needs L / Bk == d)."""
    assert L // Bk == d and L % Bk == 0
    rng = np.random.default_rng([seed, 7779])
    k = np.zeros((1, H, L, d), dtype=np.float32)
    for h in range(H):
        for b in range(L // Bk):
            blk = np.zeros((Bk, d), dtype=np.float32)
            for c in range(d):
                j = int(rng.integers(0, Bk // 2 + 1))
                idx = rng.permutation(Bk)[: 2 * j]
                blk[idx[:j], c] = 1.0
                blk[idx[j:], c] = -1.0
            blk[:, b] += 1.0
            k[0, h, b * Bk:(b + 1) * Bk] = blk
    return k


def exact_family_block(rng: np.random.Generator, d: int = 64, groups: int = 8, rows_per_group: int = 8,
                       families: Optional[int] = None) -> np.ndarray:
    """One candidate query block [groups * rows_per_group, d] of small integers for the second
    integer workload: ``groups`` groups of identical rows, randomly interleaved.

    The groups fall into ``families`` (1, 2 or 4; random if None) of equal size.  All groups of a
    family share one active pattern: a multiset of exponents on random channels, made from {E}
    (E ~ U{0..6}) by repeatedly splitting a term e into two terms e - 1 (depth <= 10), so that
    sum 2^a is a power of two; the other channels hold -80 - 16 u with u in {0, 1} drawn per
    group and channel, which separates the groups of a family.  Values are integers with
    |x| <= 96, exact in bf16.  Whether a block's selection stays exactly representable depends
    on how the clustering merges the groups, so callers keep only the blocks that pass such a
    check.
    """
    if families is None:
        families = int(rng.choice([1, 2, 4]))
    assert groups % families == 0
    per = groups // families
    centres = []
    for _f in range(families):
        E = int(rng.integers(0, 7))
        terms = [E]
        for _ in range(int(rng.integers(0, 16))):
            cand = [t for t in range(len(terms)) if terms[t] > E - 10]
            if not cand:
                break
            t = cand[int(rng.integers(0, len(cand)))]
            e = terms.pop(t)
            terms += [e - 1, e - 1]
        chans = rng.choice(d, size=len(terms), replace=False)
        active = np.zeros(d, dtype=bool)
        active[chans] = True
        for _g in range(per):
            c = (-80.0 - 16.0 * rng.integers(0, 2, size=d)).astype(np.float32)
            c[chans] = np.asarray(terms, dtype=np.float32)
            centres.append(c)
    rows = np.repeat(np.stack(centres), rows_per_group, axis=0)
    return rows[rng.permutation(rows.shape[0])]
