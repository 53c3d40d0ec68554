"""Throughput of the AB-Attention hot path on one MI355X.

One step = block selection (KV block means, in-block k-means, block scoring, SIP capping /
Philox draws / compaction) followed by gather-attention over the selected blocks, on the
Wan2.1-14B-shaped 720p workload (B=1, H=40, grid 21x45x80 = 75 600 tokens, d=128, query
block 128, KV block 16, IBCS 4 clusters x 3 k-means steps) with synthetic seeded inputs
already resident in HBM.

Prints one JSON line: value = dense-equivalent attention TFLOP/s of the whole step
(4 B H L^2 d per step / step time).  ``roofline`` covers the dominant kernel (gather-attention):
its algorithmic MFMA FLOPs (4 n_q d per kept key per row) over its average launch time, measured
with HIP events on the stream it runs on.  ``cpu_baseline`` times the fp64 oracle on a bounded
sample of the same workload on the host cores.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=(2, 3, 4),
                    help="2: Wan2.1-1.3B-shaped 480p, 3: Wan2.1-14B-shaped 720p (default), "
                         "4: HunyuanVideo-shaped 720p")
    ap.add_argument("--keep", type=float, default=None, help="block budget (default: 9.5%% for config 3, "
                                                                  "else the workload's own)")
    ap.add_argument("--kv-block", type=int, default=16)
    ap.add_argument("--heads", type=int, default=0, help="restrict H (0 = all 40)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=1920)
    ap.add_argument("--cpu-single-rows", type=int, default=240, help="rows of the one-thread oracle sample")
    ap.add_argument("--kernels-once", action="store_true",
                    help="for counter collection: one selection, two sparse attentions and one dense attention, "
                         "then exit (no JSON line)")
    ap.add_argument("--extra", action="store_true", help="also time the dense kernel, the FP8 variant and per-cluster lists")
    ap.add_argument("--ablation", action="store_true",
                    help="instead of the JSON line: accuracy and time of SIP / top-k / block-size / prior-art "
                         "selection against dense attention, as a markdown table")
    return ap.parse_args()


def ablation(args):
    """Error of the estimator against dense attention (rel-L2 over the whole output) and the time of
    selection and attention, for: SIP at three budgets and three seeds, top-k truncation at the same
    budgets, the KV block size at a 10% budget, and the coarse prior-art arm (one mean query per block,
    top-k, 64- and 128-key blocks, the latter a whole 128 x 128 tile).  On three inputs: the workload
    as generated (its 10x-norm outlier tokens act as attention sinks: about one effective key per
    query), and the same recipe without outlier tokens with queries scaled by 1/4 and by 1/8 (more
    diffuse attention); the effective number of keys per query (exp of the softmax entropy, mean
    over sampled rows) is printed for each.
    Times are HIP-event means over 5 launches after 2 warm-ups."""
    import numpy as np
    import torch

    import block_sparse_attention_34_amd as absa
    from workloads import gen_config

    from workloads import CONFIGS, gen_fourier_heads

    wl = gen_config(3, kv_block=16)
    dev = lambda x: torch.from_numpy(x).cuda().to(torch.bfloat16)  # noqa: E731
    stream = torch.cuda.current_stream()
    dense_flops = 4.0 * wl.B * wl.H * float(wl.L) ** 2 * wl.d

    def timed(fn, n=5):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    p16 = absa.Problem(wl.B, wl.H, wl.L, wl.d, wl.T, wl.Hs, wl.Ws, wl.q_block, 16)
    o_dense = torch.empty((p16.B, p16.H, p16.L, p16.d), dtype=torch.float32, device="cuda")
    o = torch.empty_like(o_dense)
    sample = np.random.default_rng(12345).choice(p16.rows, 16, replace=False)
    print(f"Workload: {wl.name} (B={wl.B}, H={wl.H}, L={wl.L}, d={wl.d}, Bq={wl.q_block}).\n")
    spec = CONFIGS[3]
    for outliers, temp in ((True, 1.0), (False, 0.25), (False, 0.125)):
        # same recipe and seed, with or without the outlier tokens
        qn, kn, vn = gen_fourier_heads(spec.T, spec.Hs, spec.Ws, spec.d, spec.modes, spec.noise_std, outliers,
                                       3, list(range(spec.H)))
        sh = (1, spec.H, spec.L, spec.d)
        q0, k, v = dev(qn.reshape(sh)), dev(kn.reshape(sh)), dev(vn.reshape(sh))
        del qn, kn, vn
        q = (q0.float() * temp).to(torch.bfloat16).contiguous()
        t_dense = timed(lambda: absa.dense(p16, q, k, v, out=o_dense))
        ref_norm = float(torch.linalg.vector_norm(o_dense))
        eff = []
        for r in sample:
            bh, qb = divmod(int(r), p16.nq)
            qs = q[0, bh, qb * wl.q_block: min((qb + 1) * wl.q_block, wl.L)].float()
            pr = torch.softmax(qs @ k[0, bh].float().T / math.sqrt(wl.d), dim=1)
            eff.append(float(torch.exp(-(pr * torch.log(pr + 1e-30)).sum(1)).mean()))
        rows = []

        def run(label, Bk, keep, mode, seed, clusters=4, steps=0):
            p = absa.Problem(wl.B, wl.H, wl.L, wl.d, wl.T, wl.Hs, wl.Ws, wl.q_block, Bk)
            lists = absa.alloc_lists(p)
            ws = torch.empty(absa.select_workspace_bytes(p, keep, clusters=clusters, kmeans_steps=steps, mode=mode),
                             dtype=torch.uint8, device="cuda")
            sel = lambda: absa.select(p, q, k, keep, clusters=clusters, kmeans_steps=steps,  # noqa: E731
                                      seed=seed, mode=mode, lists=lists, workspace=ws)
            t_sel = timed(sel)
            t_att = timed(lambda: absa.attend_balanced(p, q, k, v, lists, out=o))
            err = float(torch.linalg.vector_norm(o - o_dense)) / ref_norm
            kept = float(lists.count.double().mean()) / p.nk
            rows.append((label, Bk, keep, seed, clusters, kept, err, t_sel, t_att))
            print(f"[ablation] temp {temp} {label} Bk={Bk} keep={keep} seed={seed} C={clusters}: "
                  f"rel-L2 {err:.4e} select {t_sel:.2f} ms attend {t_att:.2f} ms", file=sys.stderr, flush=True)

        for keep in (0.08, 0.095, 0.11):
            for seed in (0, 1, 2):
                run("IBCS+SIP", 16, keep, "sip", seed)
            run("IBCS+top-k", 16, keep, "topk", 0)
        for Bk in (16, 32, 64, 128):
            run("IBCS+SIP", Bk, 0.10, "sip", 0)
            run("IBCS+top-k", Bk, 0.10, "topk", 0)
        for Bk in (64, 128):
            run("mean query+top-k (prior art)", Bk, 0.10, "topk", 0, clusters=1)
            run("mean query+SIP", Bk, 0.10, "sip", 0, clusters=1)
        # the IBCS knobs at Bk 16, keep 9.5%: cluster count (C = 4 is above) and k-means steps
        for C in (1, 2, 8):
            run("IBCS+SIP, C sweep", 16, 0.095, "sip", 0, clusters=C)
            run("IBCS+top-k, C sweep", 16, 0.095, "topk", 0, clusters=C)
        for steps in (1, 2):
            run(f"IBCS+SIP, {steps} k-means step{'s' if steps > 1 else ''}", 16, 0.095, "sip", 0, steps=steps)
            run(f"IBCS+top-k, {steps} k-means step{'s' if steps > 1 else ''}", 16, 0.095, "topk", 0, steps=steps)

        # per-cluster lists (one SIP sample per IBCS cluster, each query over its own cluster's
        # list): the same per-cluster budget as the shared 9.5% row, and a smaller one whose
        # union is about as large as the shared list
        def run_clusters(label, keep, seed):
            cl = absa.alloc_cluster_lists(p16, 4)
            ws = torch.empty(absa.select_clusters_workspace_bytes(p16, keep), dtype=torch.uint8, device="cuda")
            t_sel = timed(lambda: absa.select_clusters(p16, q, k, keep, seed=seed, lists=cl, workspace=ws))
            t_att = timed(lambda: absa.attend_clusters(p16, q, k, v, cl, out=o))
            err = float(torch.linalg.vector_norm(o - o_dense)) / ref_norm
            kept = float(cl.count.double().mean()) / p16.nk
            rows.append((label, 16, keep, seed, 4, kept, err, t_sel, t_att))
            print(f"[ablation] temp {temp} {label} keep={keep} seed={seed}: union {kept:.4f} rel-L2 {err:.4e} "
                  f"select {t_sel:.2f} ms attend {t_att:.2f} ms", file=sys.stderr, flush=True)
            del ws

        for seed in (0, 1, 2):
            run_clusters("IBCS+SIP per cluster", 0.095, seed)
        run_clusters("IBCS+SIP per cluster", 0.035, 0)

        # FP8 path (d = 128, Bk = 16): E4M3 or INT8 QK, ExpCast P and block-mean-centred E4M3 V;
        # dense (every key) and with the SIP lists at keep 9.5%, seed 0
        lists = absa.alloc_lists(p16)
        absa.select(p16, q, k, 0.095, seed=0, lists=lists)
        o16 = torch.empty_like(o)
        absa.attend(p16, q, k, v, lists, out=o16)
        fp8_rows = []
        for qi8 in (False, True):
            ops, qws = absa.quantize_fp8(p16, q, k, v, qk_int8=qi8)
            t_q = timed(lambda: absa.quantize_fp8(p16, q, k, v, ops=ops, workspace=qws))
            t_d8 = timed(lambda: absa.attend_fp8(p16, ops, None, out=o), n=2)
            err_d8 = float(torch.linalg.vector_norm(o - o_dense)) / ref_norm
            t_s8 = timed(lambda: absa.attend_fp8(p16, ops, lists, out=o))
            err_s8 = float(torch.linalg.vector_norm(o - o_dense)) / ref_norm
            err_s8_16 = float(torch.linalg.vector_norm(o - o16) / torch.linalg.vector_norm(o16))
            fp8_rows.append(("INT8" if qi8 else "E4M3", t_q, t_d8, err_d8, t_s8, err_s8, err_s8_16))
            print(f"[ablation] temp {temp} fp8 QK {'int8' if qi8 else 'e4m3'}: quantize {t_q:.2f} ms dense "
                  f"{t_d8:.2f} ms rel-L2 {err_d8:.3e}; SIP 9.5% attend {t_s8:.2f} ms rel-L2 {err_s8:.3e} "
                  f"(vs bf16 SIP output {err_s8_16:.3e})", file=sys.stderr, flush=True)
        del ops, qws

        print(f"### {'with' if outliers else 'without'} outlier tokens, queries scaled by {temp}: effective keys per query "
              f"{np.mean(eff):.1f}; dense attention {t_dense:.2f} ms "
              f"({dense_flops / (t_dense * 1e-3) / 1e12:.0f} TFLOP/s)\n")
        print("| selection | Bk | keep | seed | C | kept fraction (per-cluster rows: of the union) | rel-L2 vs dense |"
              " select ms | attend ms | dense-equiv. TFLOP/s (select+attend) |")
        print("|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
        for (label, Bk, keep, seed, C, kept, err, ts, ta) in rows:
            print(f"| {label} | {Bk} | {keep:.3f} | {seed} | {C} | {kept:.4f} | {err:.3e} | {ts:.2f} | {ta:.2f} | "
                  f"{dense_flops / ((ts + ta) * 1e-3) / 1e12:.0f} |")
        print("\nFP8 path (ExpCast E4M3 probabilities, block-mean-centred E4M3 V; Bk 16):\n")
        print("| QK codes | quantise ms | dense: attend ms | dense: rel-L2 vs bf16 dense | SIP 9.5%: attend ms |"
              " SIP 9.5%: rel-L2 vs dense | SIP 9.5%: rel-L2 vs bf16 SIP |")
        print("|---|---:|---:|---:|---:|---:|---:|")
        for (fmt, tq, td, ed, ts8, es8, es16) in fp8_rows:
            print(f"| {fmt} | {tq:.2f} | {td:.2f} | {ed:.3e} | {ts8:.2f} | {es8:.3e} | {es16:.3e} |")
        sip = {}
        for (label, Bk, keep, seed, C, kept, err, ts, ta) in rows:
            if label == "IBCS+SIP" and Bk == 16 and keep in (0.08, 0.095, 0.11):
                sip.setdefault(keep, []).append(err)
            if label == "IBCS+SIP per cluster" and keep == 0.095:
                sip.setdefault("per-cluster 0.095", []).append(err)
        print("\nSIP rel-L2, mean +- sd over seeds 0-2 (Bk 16): " + "; ".join(
            f"keep {kp if isinstance(kp, str) else format(kp, '.3f')}: {np.mean(e):.3e} +- {np.std(e, ddof=1):.1e}"
            for kp, e in sip.items()) + "\n", flush=True)


def _logit_splits(NQ, C, BH, NKp):
    """Block-range splits of the logit product (the library's rule: at least ~2048 workgroups)."""
    mtiles = (NQ * C + 127) // 128
    ntile = NKp // 32
    nsplit = min(max((2048 + mtiles * BH - 1) // (mtiles * BH), 1), ntile)
    per = (ntile + nsplit - 1) // nsplit
    return (ntile + per - 1) // per


def attend_source_digest():
    """First 16 hex digits of the sha256 over the gather-attention kernel sources."""
    import hashlib
    h = hashlib.sha256()
    for name in ("absa_attend_tiles.h", "absa_attend.hip", "absa_attend_pp.hip"):
        h.update(open(os.path.join(ROOT, "block_sparse_attention_34_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def workload_tag(config, kv_block, keep):
    """Name of a workload's committed profiles: the default (Wan2.1-14B 720p, Bk 16, keep 9.5%)
    is "wan14b_720p", the others add the block size (if not 16) and the budget in percent."""
    base = {2: "wan13b_480p", 3: "wan14b_720p", 4: "hunyuan_720p"}[config]
    if config == 3 and kv_block == 16 and abs(keep - 0.095) < 1e-9:
        return base
    return base + (f"_bk{kv_block}" if kv_block != 16 else "") + f"_keep{keep * 100:g}"


def measured_traffic(workload_tag="wan14b_720p"):
    """HBM bytes per attend launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary of
    the workload, if it was taken on the current kernel source (else None: the kernel changed since)."""
    for stem in ("attend_kernel", "attend_select_kernels"):
        prof = os.path.join(ROOT, "profiles", f"{stem}_{workload_tag}_traffic.md")
        try:
            fields = dict(line.split(": ", 1) for line in open(prof).read().splitlines() if ": " in line
                          and line.split(": ", 1)[0] in ("traffic_bytes_per_launch", "attend_source_sha256_16"))
            if fields.get("attend_source_sha256_16") == attend_source_digest():
                return int(fields["traffic_bytes_per_launch"])
        except (OSError, ValueError, KeyError):
            pass
    return None


def live_gfx_clock_ghz(launch, n_launch):
    """Graphics clock (GHz) that AMD SMI reports while ``launch`` runs back to back ``n_launch`` times:
    the mean over the XCDs' current clocks, averaged over the metric table's refreshes that come after
    the launches were queued (the table refreshes about once a second, so the launches should cover a
    few seconds); None if AMD SMI is not available or no refresh fell inside the load.  Runs outside any
    timed region."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception:
        return None
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) != 1:
            return None
        h = handles[0]
        readings, done = {}, threading.Event()
        first = []

        def poll():
            while not done.is_set():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    stamp = m.get("system_clock_counter")
                    per_xcd = m.get("current_gfxclks")
                    vals = [x for x in per_xcd if isinstance(x, (int, float)) and 0 < x < 10000] \
                        if isinstance(per_xcd, (list, tuple)) else []
                    if not vals and isinstance(m.get("current_gfxclk"), (int, float)):
                        vals = [m["current_gfxclk"]]
                    if vals and isinstance(stamp, (int, float)):
                        if not first:
                            first.append(stamp)  # the table as it stood before the load
                        elif stamp != first[0]:
                            readings[stamp] = sum(vals) / len(vals)
                except Exception:
                    pass
                done.wait(0.005)

        torch.cuda.synchronize()
        th = threading.Thread(target=poll, daemon=True)
        th.start()
        for _ in range(n_launch):
            launch()
        torch.cuda.synchronize()
        done.set()
        th.join()
        if not readings:
            return None
        return sum(readings.values()) / len(readings) / 1000.0
    except Exception:
        return None
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def _oracle_sample(wl, keep, kv_block, rows):
    """Seconds the fp64 oracle takes for S1 of one head and for S2-S6 of ``rows``."""
    import numpy as np
    import oracle as O
    Bq, d = wl.q_block, wl.d
    NQ = O.num_blocks(wl.L, Bq)
    sigma = 1.0 / math.sqrt(d)
    keep32 = float(np.float32(keep))
    t0 = time.perf_counter()
    O.kv_block_means(wl.k[0, rows[0] // NQ], kv_block)
    t_s1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    res = O.select(wl.q, wl.k, Bq, kv_block, keep32, seed=0, rows=rows)
    lists = {int(r): (res.kv_idx[i], res.inv_pi[i]) for i, r in enumerate(res.rows)}
    O.attend_rows(wl.q, wl.k, wl.v, Bq, kv_block, lists, sigma)
    t_rows = time.perf_counter() - t0
    # the per-row timing above includes S1 of each sampled head once; remove it
    heads = len(set(r // NQ for r in rows))
    per_row = max(t_rows - heads * t_s1, 1e-9) / len(rows)
    return t_s1, t_rows, per_row


def cpu_baseline(wl, keep, kv_block, nrows, nrows_single):
    """fp64 oracle on a bounded sample: S1 for one head plus S2-S6 for ``nrows`` seeded rows,
    extrapolated to the whole workload; then the same on ``nrows_single`` rows with one thread."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threadpool_limits = None
        threads = len(os.sched_getaffinity(0))
    NQ = O.num_blocks(wl.L, wl.q_block)
    BH = wl.B * wl.H
    dense_flops = 4.0 * wl.B * wl.H * float(wl.L) ** 2 * wl.d
    rng = np.random.default_rng(12345)
    rows = sorted(int(r) for r in rng.choice(BH * NQ, size=nrows, replace=False))
    t_s1, t_rows, per_row = _oracle_sample(wl, keep, kv_block, rows)
    full_s = BH * t_s1 + BH * NQ * per_row
    out = {"value": dense_flops / full_s / 1e12, "unit": "dense-equivalent TFLOP/s", "cores": int(threads),
           "kind": "oracle", "rows_per_s": 1.0 / per_row,
           "sample": (f"fp64 NumPy oracle: KV block means of one head ({t_s1:.2f} s) and selection + "
                      f"1/pi-weighted attention of {len(rows)} seeded rows ({t_rows:.2f} s) of the "
                      f"same workload, extrapolated to {BH} heads x {NQ} query blocks "
                      f"({full_s:.0f} s)")}
    if threadpool_limits is not None and nrows_single > 0:
        rows1 = rows[:nrows_single]
        with threadpool_limits(limits=1):
            t1_s1, t1_rows, per_row1 = _oracle_sample(wl, keep, kv_block, rows1)
        full1 = BH * t1_s1 + BH * NQ * per_row1
        out["single_thread"] = {"value": dense_flops / full1 / 1e12, "rows_per_s": 1.0 / per_row1, "cores": 1,
                                "sample": f"the first {len(rows1)} of those rows on one thread ({t1_rows:.2f} s), "
                                          f"extrapolated the same way ({full1:.0f} s)"}
    return out


def main():
    args = parse()
    if args.gpus == 1 and args.ablation:
        ablation(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (heads shard "
              f"across GPUs with no communication; run one process per GPU).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_attention_34_amd as absa
    from workloads import gen_config

    from workloads import CONFIGS
    heads = list(range(args.heads)) if args.heads else None
    if args.keep is None:
        args.keep = 0.095 if args.config == 3 else CONFIGS[args.config].keep[0]
    t0 = time.perf_counter()
    wl = gen_config(args.config, heads=heads, kv_block=args.kv_block)
    print(f"[bench] generated {wl.name} H={wl.H} L={wl.L} in {time.perf_counter() - t0:.1f}s",
          file=sys.stderr, flush=True)
    p = absa.Problem(wl.B, wl.H, wl.L, wl.d, wl.T, wl.Hs, wl.Ws, wl.q_block, args.kv_block)
    dev = lambda x: torch.from_numpy(x).cuda().to(torch.bfloat16)  # noqa: E731
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    lists = absa.alloc_lists(p)
    o = torch.empty((p.B, p.H, p.L, p.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(absa.select_workspace_bytes(p, args.keep), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    # 64-query blocks: adjacent blocks share one 128-query row of the two-row kernel (absa_attend_pairs);
    # 128-query blocks: the two-row kernel on its persistent grid (absa_attend_balanced)
    pairs = p.q_block == 64
    pws = torch.empty(absa.attend_pairs_workspace_bytes(p), dtype=torch.uint8, device="cuda") if pairs else \
        torch.empty(absa.attend_balanced_workspace_bytes(), dtype=torch.uint8, device="cuda")

    def attend(lst, out):
        if pairs:
            absa.attend_pairs(p, q, k, v, lst, out=out, workspace=pws)
        else:
            absa.attend_balanced(p, q, k, v, lst, out=out, workspace=pws)

    def step():
        absa.select(p, q, k, args.keep, seed=0, lists=lists, workspace=ws)
        attend(lists, o)

    if args.kernels_once:
        step()
        attend(lists, o)
        absa.dense(p, q, k, v, out=o)
        torch.cuda.synchronize()
        print("[bench] kernels-once done", file=sys.stderr, flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        absa.select(p, q, k, args.keep, seed=0, lists=lists, workspace=ws)
        ev[s][1].record(stream)
        attend(lists, o)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    sel_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in range(args.steps)]
    att_ms = [ev[s][1].elapsed_time(ev[s][2]) for s in range(args.steps)]
    step_ms = ev[0][0].elapsed_time(ev[-1][2]) / args.steps
    print(f"[bench] timed {args.steps} steps: {step_ms:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f})",
          file=sys.stderr, flush=True)

    # work the attend launch did, from the lists it consumed
    count = lists.count.long()
    NQ, NK, L, d, Bq, Bk = p.nq, p.nk, p.L, p.d, p.q_block, p.kv_block
    rows = torch.arange(p.rows, device="cuda")
    nq_valid = torch.clamp(L - (rows % NQ) * Bq, max=Bq).double()
    cap = lists.kv_idx.shape[1]
    mask = torch.arange(cap, device="cuda")[None, :] < count[:, None]
    blk = lists.kv_idx.long()
    nk_valid = torch.clamp(L - blk * Bk, max=Bk).double() * mask
    kept_keys = nk_valid.sum(dim=1)
    alg_flops = float((4.0 * nq_valid * d * kept_keys).sum())
    # the attention kernel runs 128-query rows 2p and 2p + 1 together, max(T, T') 64-key steps
    # each (with 64-query blocks, the rows are the pairs' union lists the timed calls left)
    if pairs:
        rows128 = p.B * p.H * (-(-L // 128))
        tiles = (pws[: rows128 * 4].view(torch.int32).long() * Bk + 63) // 64
    else:
        tiles = (count * Bk + 63) // 64
    tp = torch.nn.functional.pad(tiles, (0, tiles.numel() % 2)).view(-1, 2)
    exec_tiles = 2.0 * float(tp.max(dim=1).values.double().sum())
    exec_flops = 4.0 * 128 * 64 * d * exec_tiles
    alg_bytes = float(kept_keys.sum()) * 4 * d  # K + V bf16 gathered per kept key
    dense_flops = 4.0 * p.B * p.H * float(L) ** 2 * d
    att_avg = sum(att_ms) / len(att_ms)
    sel_avg = sum(sel_ms) / len(sel_ms)
    achieved = alg_flops / (att_avg * 1e-3) / 1e12
    line = {
        "metric": "dense-equivalent attention TFLOP/s + executed-MFMA % of bf16 peak, 1 GPU",
        "value": dense_flops / (step_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Fourier-mode Q/K with outlier tokens, N(0,1) V)",
        "config": {"workload": wl.name, "B": p.B, "H": p.H, "L": L, "d": d, "grid": [wl.T, wl.Hs, wl.Ws],
                   "q_block": Bq, "kv_block": Bk, "keep": args.keep, "clusters": 4, "kmeans_steps": 3,
                   "selection": "IBCS + SIP", "seed": 0,
                   "attend": "pairs of 64-query blocks" if pairs else "two-row kernel, persistent grid"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic(workload_tag(args.config, Bk, args.keep))
                     if not args.heads else None},
        "attend_ms": att_avg,
        "select_ms": sel_avg,
        "attend_dense_equiv_tflops": dense_flops / (att_avg * 1e-3) / 1e12,
        "executed_mfma_frac": exec_flops / (att_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "kept_fraction": float(count.double().mean()) / NK,
        "gather_GBs": alg_bytes / (att_avg * 1e-3) / 1e9,
        "attend_ms_median_min": [statistics.median(att_ms), min(att_ms)],
        "select_ms_median_min": [statistics.median(sel_ms), min(sel_ms)],
    }
    # the attention kernel's fraction of the bf16 peak at the clock it runs at under this load: the
    # graphics clock AMD SMI reports while the same launch repeats (after the timed region), else the
    # GRBM_GUI_ACTIVE clock of the committed counter summary of the same sources
    clk = live_gfx_clock_ghz(lambda: attend(lists, o), max(4, int(round(3000.0 / max(att_avg, 1e-3)))))
    clk_src = "AMD SMI current_gfxclk, mean over the XCDs and the metric refreshes during 3 s of repeated " \
              "attend launches after the timed region"
    if clk:
        peak_clk = MFMA_BF16_PEAK_TFLOPS * clk / 2.4
        line["roofline_at_measured_clock"] = {"clock_GHz": clk, "source": clk_src, "peak": peak_clk,
                                              "frac": achieved / peak_clk,
                                              "executed_frac": exec_flops / (att_avg * 1e-3) / 1e12 / peak_clk}
    # the selection kernel by kernel (HIP events between its launches), with the bytes each must
    # move at least: its inputs read once and its outputs written once
    prof = [absa.select_profile(p, q, k, args.keep, seed=0, lists=lists, workspace=ws)[1] for _ in range(3)]
    C, BH, rows_n = 4, p.B * p.H, p.rows
    NKp, NKs = -(-NK // 64) * 64, -(-NK // 4) * 4
    nsplit = _logit_splits(NQ, C, BH, NKp)
    qk_bytes = BH * L * d * 2
    kbh_bytes = BH * NKp * d * 4
    mu_bytes = rows_n * C * (d + 1) * 4
    mz_bytes = rows_n * C * nsplit * 8
    s_bytes = rows_n * NKs * 4
    list_bytes = float(count.sum()) * 8 + rows_n * 4
    alg = {"block means": qk_bytes + kbh_bytes, "k-means": qk_bytes + mu_bytes,
           "logit normalisers": kbh_bytes + mu_bytes + mz_bytes,
           "scores": kbh_bytes + mu_bytes + mz_bytes + s_bytes, "sampling": s_bytes + list_bytes}
    sk = {}
    for name in absa.SELECT_KERNELS:
        t = sum(pr[name] for pr in prof) / len(prof)
        sk[name] = {"ms": t, "bytes": alg[name], "GBs": alg[name] / (t * 1e-3) / 1e9,
                    "hbm_frac": alg[name] / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}
    line["select_kernels"] = sk
    line["select_alg_bytes"] = 2 * qk_bytes + list_bytes
    # accuracy of the timed step's output against dense attention, and of top-k lists of the same
    # budget (after the timed region)
    o_dense = torch.empty_like(o)
    absa.dense(p, q, k, v, out=o_dense)
    ref_norm = float(torch.linalg.vector_norm(o_dense))
    o_tk = torch.empty_like(o)
    lists_tk = absa.alloc_lists(p)
    absa.select(p, q, k, args.keep, seed=0, mode="topk", lists=lists_tk, workspace=ws)
    attend(lists_tk, o_tk)
    line["rel_l2_vs_dense"] = {"sip": float(torch.linalg.vector_norm(o - o_dense)) / ref_norm,
                               "topk": float(torch.linalg.vector_norm(o_tk - o_dense)) / ref_norm}
    del o_dense, o_tk, lists_tk
    if args.extra:
        for _ in range(2):
            absa.dense(p, q, k, v, out=o)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            absa.dense(p, q, k, v, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / 3
        line["dense_ms"] = dms
        line["dense_mfma_frac"] = dense_flops / (dms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
        dclk = live_gfx_clock_ghz(lambda: absa.dense(p, q, k, v, out=o), max(3, int(round(3000.0 / max(dms, 1e-3)))))
        if dclk:
            line["dense_clock_GHz"] = dclk
        if Bq == 128:
            # the sparse kernel over lists of every block in order, against the dense kernel (the
            # same tiles): the cost of the list decoding alone; then over the timed SIP lists (the
            # gathered order as well).  Time per 128-query row and 64-key tile.
            lists_all = absa.alloc_lists(p)
            ws_all = torch.empty(absa.select_workspace_bytes(p, 1.0, mode="all"), dtype=torch.uint8, device="cuda")
            absa.select(p, q, k, 1.0, mode="all", lists=lists_all, workspace=ws_all)
            attend(lists_all, o)
            e0.record(stream)
            for _ in range(2):
                attend(lists_all, o)
            e1.record(stream)
            torch.cuda.synchronize()
            all_tiles = float(((lists_all.count.long() * Bk + 63) // 64).double().sum())
            row_tiles_dense = float(p.rows * (-(-L // 64)))
            line["row_tile_ns"] = {"dense": dms * 1e6 / row_tiles_dense,
                                   "sparse_all_blocks": e0.elapsed_time(e1) / 2 * 1e6 / all_tiles,
                                   "sparse_sip": att_avg * 1e6 / exec_tiles}
            del lists_all, ws_all
        if Bk == 16 and wl.d == 128 and Bq == 128:
            # the FP8 variant of the attention step on the same lists (not the headline: lower precision)
            for qi8 in (False, True):
                ops, qws = absa.quantize_fp8(p, q, k, v, qk_int8=qi8)
                o8 = torch.empty_like(o)
                for _ in range(2):
                    absa.attend_fp8(p, ops, lists, out=o8)
                e0.record(stream)
                for _ in range(5):
                    absa.quantize_fp8(p, q, k, v, ops=ops, workspace=qws)
                e1.record(stream)
                torch.cuda.synchronize()
                tq = e0.elapsed_time(e1) / 5
                e0.record(stream)
                for _ in range(5):
                    absa.attend_fp8(p, ops, lists, out=o8)
                e1.record(stream)
                torch.cuda.synchronize()
                tag = "int8qk" if qi8 else "e4m3"
                line[f"fp8_{tag}_attend_ms"] = e0.elapsed_time(e1) / 5
                line[f"fp8_{tag}_quantize_ms"] = tq
                del ops, qws, o8
            # per-cluster lists (C = 4, the same keep per cluster): selection and attention
            cl = absa.alloc_cluster_lists(p, 4)
            cws = torch.empty(absa.select_clusters_workspace_bytes(p, args.keep), dtype=torch.uint8, device="cuda")
            oc = torch.empty_like(o)
            absa.select_clusters(p, q, k, args.keep, seed=0, lists=cl, workspace=cws)
            absa.attend_clusters(p, q, k, v, cl, out=oc)
            e0.record(stream)
            for _ in range(3):
                absa.select_clusters(p, q, k, args.keep, seed=0, lists=cl, workspace=cws)
            e1.record(stream)
            torch.cuda.synchronize()
            line["clusters_select_ms"] = e0.elapsed_time(e1) / 3
            e0.record(stream)
            for _ in range(3):
                absa.attend_clusters(p, q, k, v, cl, out=oc)
            e1.record(stream)
            torch.cuda.synchronize()
            line["clusters_attend_ms"] = e0.elapsed_time(e1) / 3
            line["clusters_union_fraction"] = float(cl.count.double().mean()) / p.nk
            del cl, cws, oc
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.keep, args.kv_block, args.cpu_sample_rows,
                                            args.cpu_single_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
