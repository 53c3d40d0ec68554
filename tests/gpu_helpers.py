"""Shared helpers for the GPU parity tests (imported by test modules, collects no tests)."""
import numpy as np

import oracle as O
from workloads import Workload

# Tolerances for GPU outputs against the fp64 oracle fed the same lists: bf16 inputs, bf16
# probabilities in the PV product, fp32 accumulation.
MAX_ABS = 1e-2
REL_L2 = 5e-3
AGREE = 0.999


def dev(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch.bfloat16)


def problem(wl: Workload, kv_block=None, q_block=None, scale=0.0, out_bf16=False):
    import block_sparse_attention_34_amd as absa
    return absa.Problem(wl.B, wl.H, wl.L, wl.d, wl.T, wl.Hs, wl.Ws, q_block or wl.q_block,
                        kv_block or wl.kv_block, scale, out_bf16)


def keep32(keep: float) -> float:
    """The library takes keep as fp32; the oracle is fed the same value."""
    return float(np.float32(keep))


def lists_to_host(lists):
    return (lists.count.cpu().numpy(), lists.kv_idx.cpu().numpy(), lists.inv_pi.cpu().numpy())


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    max_abs = float(np.abs(got - ref).max()) if got.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)) if got.size else 0.0
    return max_abs, rel


def assert_close(got, ref, what=""):
    max_abs, rel = errors(got, ref)
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    return max_abs, rel


def oracle_rows_from_gpu_lists(wl: Workload, Bq, Bk, count, kv_idx, inv_pi, rows, sigma):
    lists = {int(r): (kv_idx[r, :count[r]], inv_pi[r, :count[r]]) for r in rows}
    return O.attend_rows(wl.q, wl.k, wl.v, Bq, Bk, lists, sigma)


def gpu_rows(o: np.ndarray, wl: Workload, Bq: int, rows):
    NQ = -(-wl.L // Bq)
    out = {}
    for r in rows:
        bh, i = divmod(int(r), NQ)
        b, h = divmod(bh, wl.H)
        out[int(r)] = o[b, h, i * Bq: min(wl.L, (i + 1) * Bq)]
    return out


def decision_agreement(count, kv_idx, res: O.SelectResult, NK: int):
    """1 - (#(row, b) kept by exactly one side) / (rows * NK) over the oracle's rows."""
    diff = 0
    for r_i, r in enumerate(res.rows):
        g = np.zeros(NK, bool)
        g[kv_idx[r, :count[r]]] = True
        o = np.zeros(NK, bool)
        o[res.kv_idx[r_i]] = True
        diff += int((g ^ o).sum())
    return 1.0 - diff / (len(res.rows) * NK)


def sample_rows(NQ: int, BH: int, n: int, seed: int = 12345, tails: int = 4):
    rng = np.random.default_rng(seed)
    rows = set(int(x) for x in rng.choice(BH * NQ, size=min(n, BH * NQ), replace=False))
    for bh in rng.choice(BH, size=min(tails, BH), replace=False):
        rows.add(int(bh) * NQ + NQ - 1)  # the head's tail query block
    return sorted(rows)


def assert_selection_bit_exact(absa, wl: Workload, C: int, Tk: int, mode: int, seed: int, stream_id: int = 3):
    """absa_select on an integer workload (alpha 1, keep 25%) against the oracle: counts, indices,
    weights and probabilities bit-identical, and the workspace's block means, centroids, cluster
    sizes and scores equal to the oracle's intermediates."""
    import torch
    p = problem(wl)
    lists, pi, ws = absa.select(p, dev(wl.q), dev(wl.k), 0.25, clusters=C, kmeans_steps=Tk,
                                select_scale_log2=1.0, seed=seed, stream_id=stream_id, mode=mode, want_pi=True)
    torch.cuda.synchronize()
    count, kv, w = lists_to_host(lists)
    res = O.select(wl.q, wl.k, wl.q_block, wl.kv_block, 0.25, C=C, Tk=Tk, alpha=1.0, seed=seed, stream=stream_id,
                   mode=mode, keep_intermediates=True)
    np.testing.assert_array_equal(count, res.count)
    for r in range(p.rows):
        np.testing.assert_array_equal(kv[r, :count[r]], res.kv_idx[r])
        np.testing.assert_array_equal(w[r, :count[r]].view(np.uint32), res.inv_pi[r].view(np.uint32))
    np.testing.assert_array_equal(pi.cpu().numpy().view(np.uint32), res.pi_hat.view(np.uint32))
    offs = absa.workspace_layout(p, 0.25, C, Tk, mode)
    wsn = ws.cpu().numpy()
    BH, NK, d = wl.B * wl.H, p.nk, wl.d
    NKp = -(-NK // 64) * 64
    kbarT = wsn[offs[0]: offs[0] + BH * d * NKp * 4].view(np.float32).reshape(BH, d, NKp)
    np.testing.assert_array_equal(kbarT[:, :, :NK].transpose(0, 2, 1), res.kbar.astype(np.float32))
    mu = wsn[offs[1]: offs[1] + p.rows * C * d * 4].view(np.float32).reshape(p.rows, C, d)
    np.testing.assert_array_equal(mu, res.mu.astype(np.float32))
    nj = wsn[offs[2]: offs[2] + p.rows * C * 4].view(np.int32).reshape(p.rows, C)
    np.testing.assert_array_equal(nj, res.counts)
    NKs = -(-NK // 4) * 4    # score rows are padded to a multiple of 4 entries (zeros)
    s = wsn[offs[3]: offs[3] + p.rows * NKs * 4].view(np.float32).reshape(p.rows, NKs)
    np.testing.assert_array_equal(s[:, :NK], res.scores.astype(np.float32))
    assert not s[:, NK:].any()
    return count, kv, w
