"""Benchmark of the top-k sparse decode attention path on one MI355X.

Workload (default): the Llama-3.1-8B-shaped decode step -- batch 16, 32 query
/ 8 KV heads, head_dim 128, bf16 KV cache of 32768 tokens per sequence, exact
top-k per (sequence, KV head) at 50x sparsity (k = 655).  One step is one pass
of the whole hot path through the C ABI:
    sa_select (exact scoring fused with a per-part top-k, then the merge)
    -> sa_sparse_decode (gather + split-K attend).
Queries rotate over 8 pre-generated variants and the steps over 8 device
copies of the cache (2.15 GB each, all resident in HBM before timing starts;
--kv-replicas), so consecutive steps select different tokens and no step
finds the previous step's rows in cache.

Timing: W untimed warmup steps, then K timed steps bracketed by
torch.cuda.synchronize().  Each step is captured once per query variant as a
HIP graph of its three launches and replayed (a serving loop's form; --eager
times plain launches instead); the bench checks that a replay selects and
attends exactly as an eager step.  A separate pass of eager steps with HIP
events recorded on the launch stream between the two calls gives each call's
average duration.

Prints ONE JSON line.  `value` is the step's achieved HBM bandwidth
(algorithmic bytes of selection + attend per step / time per step);
`steps_per_s` is the decode-step rate; `roofline` is the dominant unit (the
sa_select call: its fused kernel and merge); `kernels` holds each unit's
bytes, time and fraction of the 8 TB/s peak, including the gather-attend
alone, the unfused selection (sa_score then sa_topk on the same inputs) and a
dense decode over the same cache for comparison; `stream_read` is the
device's streaming read rate (sa_stream_read over 8 GiB), and the step's and
the dominant unit's rates are also given as fractions of it.  `cpu_baseline` times the
CPU oracle on a bounded sample of the same step (rows of the batch), scaled
to a full step.

Other modes (each prints its own JSON line): --sweep (full step with four
selection front ends against dense decode at 2x-500x on the llama32k and
batch128k shapes), --hylra (layer-reuse plans over 8 layers), --offload
(selected blocks fetched from a pinned host cache), --nscale (32K-128K
tokens at fixed k), --indexer1m (the 1M-token 8-layer mixed plan),
--block61k (block selection and reuse on the device); --profile (a short
run for rocprofv3), --traffic and --summarize (reports from its results).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E peak, GB/s
N_QVAR = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama32k")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="bound on the oracle's CPU time for cpu_baseline (0 disables)")
    p.add_argument("--dense-steps", type=int, default=20)
    p.add_argument("--kv-replicas", type=int, default=8,
                   help="copies of the K/V cache the timed steps rotate through (step i uses "
                        "copy i mod R), so a step never finds the previous step's rows in cache")
    p.add_argument("--stream-gib", type=int, default=8,
                   help="GiB read by sa_stream_read for the device's streaming read rate (0: skip)")
    p.add_argument("--eager", action="store_true",
                   help="time eager launches instead of replaying each step as a HIP graph")
    p.add_argument("--profile", action="store_true",
                   help="short run for a profiler: few steps, no dense, no cpu baseline, plus "
                        "three 1 GiB device-to-device copies that calibrate HBM byte counters")
    p.add_argument("--cold-iters", type=int, default=30,
                   help="cache-cold gather-attend launches timed after the steps (0 disables)")
    p.add_argument("--summarize", metavar="DB",
                   help="print a per-kernel summary of a rocprofv3 results database and exit")
    p.add_argument("--sweep", action="store_true",
                   help="indexer-inclusive break-even sweep: full step (exact scores or a "
                        "per-KV-head low-dim indexer, then top-k and attend) against dense decode "
                        "at 2x-500x sparsity on the llama32k and batch128k shapes; prints a table "
                        "and one JSON line")
    p.add_argument("--hylra", action="store_true",
                   help="layer-reuse policy: an 8-layer llama32k-shaped decode whose queries and "
                        "keys correlate across layers; profiles every layer, plans with the DP "
                        "planner and times all-dense, all-sparse, the fixed-jump baseline and the "
                        "planned policy; prints one JSON line")
    p.add_argument("--offload", action="store_true",
                   help="index-guided offload: block61k-shaped layers whose caches sit in pinned "
                        "host memory; times the gather of the 24 selected blocks per row over the "
                        "host link against copying the whole layer, and a 3-layer reuse pipeline "
                        "that prefetches the next layer's blocks on a second stream; one JSON line")
    p.add_argument("--nscale", action="store_true",
                   help="context-length scaling at fixed k: the llama32k shape at 32K, 64K and "
                        "128K tokens with k = 655; the gather-attend moves the same bytes at every "
                        "N while selection and dense decode grow with N; prints a table and one "
                        "JSON line")
    p.add_argument("--indexer1m", action="store_true",
                   help="one 1M-token sequence over 8 layers (32/8 heads, d 128, bf16): layers 0-1 "
                        "dense, layers 2-7 select 2048 tokens shared by the KV heads with a 4-head "
                        "64-dim indexer; times the mixed 8-layer step against all-dense and each "
                        "sparse layer's launches; prints a table and one JSON line")
    p.add_argument("--block61k", action="store_true",
                   help="block selection on the block61k workload (batch 8, 32/8 heads, d 128, bf16, "
                        "61440 tokens, 24 of 480 blocks of 128 kept): block summaries, block scores, "
                        "block top-k and the block gather-attend timed call by call, and the 4-layer "
                        "plan (SPARSE, then 3 REUSE layers) against all-dense; one JSON line")
    p.add_argument("--theta", type=float, default=0.35,
                   help="overlap threshold of the layer-reuse planner (--hylra)")
    p.add_argument("--traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                   help="print the calibrated HBM traffic per dispatch from two rocprofv3 --pmc "
                        "runs of `bench.py --profile` (FETCH_SIZE, then WRITE_SIZE) and exit")
    return p.parse_args()


# ---------------------------------------------------------------------------
# rocprofv3 results -> text summary; HBM traffic from the byte counters
# ---------------------------------------------------------------------------

COPY_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "llama32k_hbm_traffic.txt")
# kernel -> (name fragment in the trace, sources whose hash the counters belong to)
# kernel -> (name fragments of its launches in the trace -- their bytes per
# dispatch add up --, sources whose hash the counters belong to)
_SEL_SRC = ["top_sparse_decode_sa_amd/csrc/select.hip", "top_sparse_decode_sa_amd/csrc/topk.hip",
            "top_sparse_decode_sa_amd/csrc/topk_core.hpp", "top_sparse_decode_sa_amd/csrc/common.hpp"]
TRAFFIC_KERNELS = {
    "select": (["select_part_kernel", "topk_reg_kernel<512, 2, true>"], _SEL_SRC),
    "sparse_attend": (["attend_sparse_kernel"], ["top_sparse_decode_sa_amd/csrc/attend.hip",
                                                 "top_sparse_decode_sa_amd/csrc/common.hpp"]),
    "score_exact": (["score_exact_kernel"], ["top_sparse_decode_sa_amd/csrc/score.hip",
                                             "top_sparse_decode_sa_amd/csrc/common.hpp"]),
    "topk": (["topk_reg_kernel<1024, 8, false>"], ["top_sparse_decode_sa_amd/csrc/topk.hip",
                                                "top_sparse_decode_sa_amd/csrc/topk_core.hpp",
                                                "top_sparse_decode_sa_amd/csrc/common.hpp"]),
}


def source_hash(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def summarize(db_path):
    """Per-kernel dispatch count and duration stats (mean, min, max, median,
    p10, p90); with counter data, the per-dispatch mean of each counter."""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, count(*), avg(end-start), min(end-start), max(end-start) "
                      "from kernels group by name order by sum(end-start) desc").fetchall()
    durs = {}
    for name, dt in db.execute("select name, end-start from kernels"):
        durs.setdefault(name, []).append(dt)
    lines = ["%-70s %6s %10s %10s %10s %10s %10s %10s" % (
        "kernel", "calls", "avg_us", "min_us", "max_us", "median_us", "p10_us", "p90_us")]
    for name, n, avg, mn, mx in rows:
        med, p10, p90 = np.percentile(np.asarray(durs[name], dtype=np.float64), [50, 10, 90])
        lines.append("%-70s %6d %10.2f %10.2f %10.2f %10.2f %10.2f %10.2f" % (
            name[:70], n, avg / 1e3, mn / 1e3, mx / 1e3, med / 1e3, p10 / 1e3, p90 / 1e3))
    try:
        pmc = db.execute("select kernel_name, counter_name, avg(value), count(*) "
                         "from counters_collection group by kernel_name, counter_name").fetchall()
    except Exception:
        pmc = []
    counters = {}
    if pmc:
        lines.append("")
        lines.append("%-70s %-14s %16s %6s" % ("kernel", "counter", "mean/dispatch", "n"))
        for name, cname, val, n in pmc:
            lines.append("%-70s %-14s %16.1f %6d" % (name[:70], cname, val, n))
            counters[(name, cname)] = val
    return "\n".join(lines), rows, counters


def provenance(clocks=False):
    """What the numbers were measured on: device name, gfx target, compute
    units, HBM size, HIP version and, if asked, the current clocks as
    rocm-smi reports them (best effort: absent if the tool is not there)."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    out = {"device": torch.cuda.get_device_name(0), "gfx": getattr(pr, "gcnArchName", None),
           "compute_units": pr.multi_processor_count,
           "hbm_gib": round(pr.total_memory / 2 ** 30, 1), "hip": torch.version.hip}
    if clocks:
        import subprocess
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                               text=True, timeout=30)
            card = next(iter(json.loads(r.stdout).values()))
            out["clocks"] = {k_: v_ for k_, v_ in card.items() if "clk" in k_.lower()}
        except Exception as e:  # the tool is absent or printed no JSON
            out["clocks"] = "unavailable (%s)" % type(e).__name__
    return out


def host_cpu():
    """Host CPU model name and logical CPU count."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cpus": os.cpu_count()}


def pmc_means(db_path, counter):
    """Per-kernel-name mean of one counter per dispatch (KiB for the byte
    counters) and the dispatch count."""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, avg(value), count(*) from counters_collection "
                      "where counter_name = ? group by kernel_name", (counter,)).fetchall()
    return {name: (val, n) for name, val, n in rows}


def db_dir_name(db_path):
    """The rocprofv3 -d folder and -o name that wrote `db_path`."""
    base = os.path.basename(db_path)
    return os.path.dirname(db_path), base[:-len("_results.db")] if base.endswith("_results.db") else base


def traffic_report(fetch_db, write_db):
    """HBM bytes per dispatch of the step's kernels.  FETCH_SIZE and
    WRITE_SIZE are scaled by what they read for the calibration copies that
    `bench.py --profile` runs (1 GiB read and 1 GiB written each)."""
    fetch = pmc_means(fetch_db, "FETCH_SIZE")
    write = pmc_means(write_db, "WRITE_SIZE")
    copy = [n for n in fetch if "copyBuffer" in n]
    if not copy:
        raise SystemExit("no calibration copy in %s" % fetch_db)
    ff = COPY_BYTES / (fetch[copy[0]][0] * 1024.0)
    wf = COPY_BYTES / (write[copy[0]][0] * 1024.0)
    c = None
    try:
        import sa_synth as S
        c = S.CONFIGS["llama32k"]
    except Exception:
        pass
    alg = step_bytes(c) if c is not None else {}
    lines = ["# HBM traffic per dispatch, calibrated byte counters",
             "#",
             "# commands (one counter per run, then this report):",
             "#   rocprofv3 --pmc FETCH_SIZE -d %s -o %s -- python -u bench.py --profile"
             % db_dir_name(fetch_db),
             "#   rocprofv3 --pmc WRITE_SIZE -d %s -o %s -- python -u bench.py --profile"
             % db_dir_name(write_db),
             "#   python bench.py --traffic %s %s" % (fetch_db, write_db),
             "# bench.py --profile runs three 1 GiB device-to-device copies that read and write",
             "# exactly 1073741824 bytes each; factor = 1073741824 / (counter KiB of a copy * 1024)",
             "#",
             "%-70s %6s %14s %14s %14s" % ("kernel", "n", "FETCH_KiB", "WRITE_KiB", "bytes(calib.)")]
    for name in sorted(fetch, key=lambda n: -fetch[n][0]):
        fk, n = fetch[name]
        wk = write.get(name, (0.0, 0))[0]
        lines.append("%-70s %6d %14.1f %14.1f %14d" % (name[:70], n, fk, wk,
                                                        round(fk * 1024 * ff + wk * 1024 * wf)))
    lines += ["", "fetch_factor: %.6f" % ff, "write_factor: %.6f" % wf]
    for key, (frags, srcs) in TRAFFIC_KERNELS.items():
        t, found = 0, True
        for frag in frags:
            names = [n for n in fetch if frag in n]
            if not names:
                found = False
                break
            name = max(names, key=lambda n: fetch[n][1])
            t += round(fetch[name][0] * 1024 * ff + write.get(name, (0.0, 0))[0] * 1024 * wf)
        if not found:
            continue
        lines.append("%s.traffic_bytes_per_launch: %d" % (key, t))
        if key in alg:
            lines.append("%s.algorithmic_bytes_per_launch: %d" % (key, alg[key]))
            lines.append("%s.traffic_over_algorithmic: %.4f" % (key, t / alg[key]))
        lines.append("%s.source_sha256_16: %s" % (key, source_hash(srcs)))
    return "\n".join(lines)


def read_traffic(kernel):
    """Measured HBM bytes per launch of `kernel`, if its counters were taken on
    the current source (null otherwise)."""
    if kernel not in TRAFFIC_KERNELS or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get(kernel + ".source_sha256_16") != source_hash(TRAFFIC_KERNELS[kernel][1]):
        return None  # the kernel changed since the counters were taken
    try:
        return int(kv[kernel + ".traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def select_candidates(rows, n, k):
    """Candidates per row of the fused exact selection (sa_select): parts of
    8192 tokens, halved (down to 256) while the grid has fewer than 512
    workgroups and the candidates stay within a quarter of the row; each part
    keeps min(k, its length).  Returns (candidates, fused)."""
    def cands(L):
        P = -(-n // L)
        return (P - 1) * min(k, L) + min(k, n - (P - 1) * L)

    L = 8192
    while L > 256 and rows * -(-n // L) < 512 and 4 * cands(L // 2) <= n:
        L //= 2
    C = cands(L)
    return C, (-(-n // L) == 1 or (C <= 32768 and 4 * C <= n))


def step_bytes(cfg):
    """Algorithmic HBM bytes of one step's kernels (each input read once,
    each output written once)."""
    B, Hq, Hkv, d, N, k = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ctx_len, cfg.k
    e = cfg.elt
    rows = B * Hkv
    q_bytes = B * Hq * d * e
    scores = rows * N * 4
    idx = rows * k * 4
    out = B * Hq * d * 4
    C, fused = select_candidates(rows, N, k)
    assert fused, "the step's selection takes the fused path"
    return {
        # sa_select: keys and queries read, (score, position) candidates
        # written and read back by the merge, the index list written
        "select": rows * N * d * e + q_bytes + 2 * rows * C * 8 + idx,
        "sparse_attend": 2 * rows * k * d * e + idx + q_bytes + out,
        "score_exact": rows * N * d * e + q_bytes + scores,
        "topk": scores + idx,
        "dense_decode": 2 * rows * N * d * e + q_bytes + out,
    }


def cpu_baseline(w, q_host, k_host, v_host, seconds):
    """Time the oracle, one BLAS thread, on whole rows of the step until
    `seconds` elapse; returns (seconds per full step, rows timed, rows)."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    c = w.cfg
    scale = O.default_scale(c.head_dim)
    rows = c.batch * c.n_kv_heads
    rows_done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        qf = O.widen(q_host[0])
        for row in range(rows):
            b, r = divmod(row, c.n_kv_heads)
            qg = qf[b, r * c.group:(r + 1) * c.group]
            kf = O.widen(k_host[b, r])
            s = O.scores_exact(qg, kf, scale)
            sel = O.topk(s, c.k)
            O.attend(qg, kf, O.widen(v_host[b, r]), sel, scale)
            rows_done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return dt * rows / rows_done, rows_done, rows


SWEEP_X = (2, 5, 10, 20, 50, 100, 200, 500)
IDX_HEADS, IDX_DIM = 4, 64


def select_fused(rows, n, k):
    """Whether sa_select takes its fused path on this shape (else it scores
    every token and runs sa_topk)."""
    return select_candidates(rows, n, k)[1]


def sweep(args):
    """Full decode step against dense decode across sparsity.

    Selection front ends feeding the same gather-attend: exact scores (every
    key row read) then sa_topk; sa_select, the same exact selection with the
    scores kept on chip (fused where the part candidates are at most a
    quarter of the row, column select_fused); and a per-KV-head lightning
    indexer, scored then sa_topk or through sa_select (keys
    projected to 64 dims, 4 indexer heads = the KV head's 4 grouped queries
    projected the same way, weights U(0,1)), which reads half the key bytes.
    The llama32k shape uses the seeded workload; batch128k (68.7
    GB of K/V) is drawn N(0,1) on the device, since only the selection sizes,
    not the values, drive the timings there."""
    import torch
    import sa_synth as S
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    reps = max(3, min(args.steps, 10))
    results = []

    def timed(fn, n, blocker=None):
        # a long kernel ahead of the timed launches lets the host queue them
        # all before the GPU reaches them, so host-side call overhead does
        # not show up as idle GPU time between short kernels
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        if blocker is not None:
            blocker()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    for shape in ("llama32k", "batch128k"):
        c = S.CONFIGS[shape]
        B, Hq, Hkv, d, N = c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.ctx_len
        G = Hq // Hkv
        log("sweep: %s inputs" % shape)
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        if shape == "llama32k":
            w = S.Workload(shape, args.seed)

            def up(x):
                t = torch.from_numpy(x)
                return (t.view(torch.bfloat16) if t.dtype == torch.uint16 else t).to(dev)

            q, kd, vd = up(w.q()), up(w.k()), up(w.v())
            data = "seeded workload (planted heavy keys)"
        else:
            q = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
            kd = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
            vd = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
            data = "N(0,1) drawn on the device"
        # per-KV-head indexer inputs (projection P [64, d], N(0, 1/d) entries)
        P = torch.randn((IDX_DIM, d), generator=gen, device=dev) / d ** 0.5
        k_idx = torch.empty((B, Hkv, N, IDX_DIM), dtype=torch.bfloat16, device=dev)
        for b in range(B):
            kb = kd[b].float() @ P.t()
            kb += 0.1 * torch.randn(kb.shape, generator=gen, device=dev)
            k_idx[b] = kb.to(torch.bfloat16)
            del kb
        q_idx = (q.float().view(B, Hkv, G, d)[:, :, :IDX_HEADS] @ P.t()).to(torch.bfloat16).contiguous()
        idx_w = torch.rand((B, Hkv, IDX_HEADS), generator=gen, device=dev)
        scores = torch.empty((B, Hkv, N), dtype=torch.float32, device=dev)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)

        def dense():
            T.sa_dense_decode(q, kd, vd, out=out)

        us_dense = timed(dense, reps)
        dense_bytes = 2 * B * Hkv * N * d * 2
        for x in SWEEP_X:
            k = N // x
            idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)

            def exact_score():
                T.sa_score(q, kd, T.SA_SCORE_EXACT, scores=scores)

            def idx_score():
                T.sa_score(q, kd, T.SA_SCORE_INDEXER_PER_KV_HEAD, q_idx=q_idx, k_idx=k_idx,
                           idx_w=idx_w, scores=scores)

            def select():
                T.sa_topk(scores, k, idx_out=idx)

            def attend():
                T.sa_sparse_decode(q, kd, vd, idx, out=out)

            def fused_select():
                T.sa_select(q, kd, k, idx_out=idx)

            def fused_idx_select():
                T.sa_select(q, kd, k, T.SA_SCORE_INDEXER_PER_KV_HEAD, idx_out=idx, q_idx=q_idx,
                            k_idx=k_idx, idx_w=idx_w)

            row = {"shape": shape, "x": x, "k": k, "dense_us": round(us_dense, 1)}
            row["exact_score_us"] = round(timed(exact_score, reps, dense), 1)
            row["indexer_us"] = round(timed(idx_score, reps, dense), 1)
            row["topk_us"] = round(timed(select, reps, dense), 1)
            row["attend_us"] = round(timed(attend, reps, dense), 1)
            row["exact_step_us"] = round(timed(lambda: (exact_score(), select(), attend()), reps,
                                               dense), 1)
            row["indexer_step_us"] = round(timed(lambda: (idx_score(), select(), attend()), reps,
                                                 dense), 1)
            row["select_us"] = round(timed(fused_select, reps, dense), 1)
            row["select_step_us"] = round(timed(lambda: (fused_select(), attend()), reps, dense), 1)
            row["select_fused"] = select_fused(B * Hkv, N, k)
            row["indexer_select_step_us"] = round(timed(lambda: (fused_idx_select(), attend()), reps,
                                                        dense), 1)
            row["attend_only_speedup"] = round(us_dense / row["attend_us"], 2)
            row["exact_step_speedup"] = round(us_dense / row["exact_step_us"], 2)
            row["indexer_step_speedup"] = round(us_dense / row["indexer_step_us"], 2)
            row["select_step_speedup"] = round(us_dense / row["select_step_us"], 2)
            row["indexer_select_step_speedup"] = round(us_dense / row["indexer_select_step_us"], 2)
            row["attend_gbps"] = round((2 * B * Hkv * k * d * 2) / row["attend_us"] / 1e3, 1)
            row["data"] = data
            results.append(row)
            log("sweep: %s x=%d done" % (shape, x))
        log("sweep: %s dense %.1f us (%.0f GB/s)" % (shape, us_dense, dense_bytes / us_dense / 1e3))
        del q, kd, vd, k_idx, q_idx, idx_w, scores, out
        torch.cuda.empty_cache()

    cols = ["shape", "x", "k", "dense_us", "exact_score_us", "indexer_us", "topk_us", "attend_us",
            "select_us", "select_fused", "exact_step_us", "select_step_us", "indexer_step_us",
            "indexer_select_step_us", "attend_only_speedup", "exact_step_speedup",
            "select_step_speedup", "indexer_step_speedup", "indexer_select_step_speedup",
            "attend_gbps"]
    print("  ".join("%12s" % c_ for c_ in cols))
    for r in results:
        print("  ".join("%12s" % r[c_] for c_ in cols))
    print(json.dumps({"sweep": "indexer-inclusive break-even", "unit": "us per step (HIP events)",
                      "rows": results, "provenance": provenance()}), flush=True)


NSCALE_N = (32768, 65536, 131072)


def nscale(args):
    """Decode step at a fixed number of selected tokens as the context grows.

    The llama32k shape (batch 16, 32/8 heads, d 128, bf16) with k = 655 at
    N = 32K, 64K and 128K.  The gather-attend reads 2*B*Hkv*k*d*2 bytes at
    every N (the sparse method's traffic does not grow with the context);
    the exact selection reads every key once and dense decode every key and
    value, so both grow linearly.  Values are N(0,1) drawn on the device:
    only the sizes drive these timings."""
    import torch
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    reps = max(3, min(args.steps, 10))
    B, Hq, Hkv, d, k = 16, 32, 8, 128, 655
    rows = []

    def timed(fn, n, blocker=None):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        if blocker is not None:
            blocker()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    for N in NSCALE_N:
        log("nscale: N=%d" % N)
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed)
        q = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
        kd = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
        vd = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev).normal_(generator=gen)
        idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)

        def dense():
            T.sa_dense_decode(q, kd, vd, out=out)

        def select():
            T.sa_select(q, kd, k, idx_out=idx)

        def attend():
            T.sa_sparse_decode(q, kd, vd, idx, out=out)

        us_dense = timed(dense, reps)
        us_sel = timed(select, reps, dense)
        us_att = timed(attend, reps, dense)
        us_step = timed(lambda: (select(), attend()), reps, dense)
        att_bytes = 2 * B * Hkv * k * d * 2
        key_bytes = B * Hkv * N * d * 2
        rows.append({
            "N": N, "k": k, "dense_us": round(us_dense, 1), "select_us": round(us_sel, 1),
            "attend_us": round(us_att, 1), "step_us": round(us_step, 1),
            "attend_bytes": att_bytes, "attend_gbps": round(att_bytes / us_att / 1e3, 1),
            "select_key_bytes": key_bytes, "select_gbps": round(key_bytes / us_sel / 1e3, 1),
            "select_fused": select_fused(B * Hkv, N, k),
            "dense_gbps": round(2 * key_bytes / us_dense / 1e3, 1),
            "step_speedup": round(us_dense / us_step, 2)})
        del q, kd, vd, idx, out
        torch.cuda.empty_cache()

    cols = ["N", "k", "dense_us", "select_us", "attend_us", "step_us", "attend_gbps",
            "select_gbps", "dense_gbps", "select_fused", "step_speedup"]
    print("  ".join("%12s" % c_ for c_ in cols))
    for r in rows:
        print("  ".join("%12s" % r[c_] for c_ in cols))
    print(json.dumps({"bench": "context-length scaling at fixed k", "unit": "us (HIP events)",
                      "config": {"workload": "llama32k shape at N = 32K, 64K, 128K, k = 655",
                                 "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d},
                      "rows": rows, "data": "N(0,1) drawn on the device (seed %d)" % args.seed,
                      "provenance": provenance()}), flush=True)


def indexer1m(args):
    """The indexer1m workload: batch 1, 32/8 heads, d 128, bf16, 1048576
    tokens, 8 layers; layers 0-1 DENSE, layers 2-7 SPARSE with the shared
    lightning indexer (4 heads of 64 dims, top-2048 shared by the 8 KV
    heads).  One 8-layer step is timed under the mixed plan and all-dense;
    one sparse layer is timed whole and call by call (indexer scores, top-k
    of the one 1M-score row, gather-attend).  Values are N(0,1) (weights
    U(0,1)) drawn on the device: the timings depend on the sizes."""
    import torch
    import sa_synth as S
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    c = S.CONFIGS["indexer1m"]
    B, Hq, Hkv, d, N, k, L = c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.ctx_len, c.k, c.n_layers
    H, Di = c.indexer_heads, c.indexer_dim
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    log("indexer1m: drawing %d layers (%.1f GB of KV)" % (L, L * c.kv_bytes() / 1e9))

    def bf(shape):
        return torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(generator=gen)

    qs = [bf((B, Hq, d)) for _ in range(L)]
    ks = [bf((B, Hkv, N, d)) for _ in range(L)]
    vs = [bf((B, Hkv, N, d)) for _ in range(L)]
    qi = [bf((B, H, Di)) for _ in range(L)]
    ki = [bf((B, N, Di)) for _ in range(L)]
    wi = [torch.rand((B, H), generator=gen, device=dev) for _ in range(L)]
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
    largs = [T.layer_args(qs[l], ks[l], vs[l], T.SA_SCORE_INDEXER, k, q_idx=qi[l], k_idx=ki[l],
                          idx_w=wi[l], out=outs[l])[0] for l in range(L)]
    ws = {m: T.WORKSPACES.get(dev, ("indexer1m", m), T.sa_layer_workspace_size(largs[0], m))
          for m in (T.SA_LAYER_DENSE, T.SA_LAYER_SPARSE)}
    idx = [torch.empty((B, k), dtype=torch.int32, device=dev) for _ in range(L)]
    mixed = [T.SA_LAYER_DENSE if m == "dense" else T.SA_LAYER_SPARSE for m in c.modes]
    T.sa_plan_validate(mixed, list(c.src))
    reps = max(3, min(args.steps, 10))

    def layer(l, m):
        T.sa_decode_layer(largs[l], m, None if m == T.SA_LAYER_DENSE else idx[l], dev, ws[m])

    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        layer(0, T.SA_LAYER_DENSE)  # queued ahead, so the host enqueues the rest in time
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    us_mixed = timed(lambda: [layer(l, mixed[l]) for l in range(L)], reps)
    us_dense8 = timed(lambda: [layer(l, T.SA_LAYER_DENSE) for l in range(L)], reps)
    us_dense = timed(lambda: layer(2, T.SA_LAYER_DENSE), reps)
    us_sparse = timed(lambda: layer(2, T.SA_LAYER_SPARSE), reps)
    scores = torch.empty((B, N), dtype=torch.float32, device=dev)
    sel = torch.empty((B, k), dtype=torch.int32, device=dev)
    us_score = timed(lambda: T.sa_score(qs[2], ks[2], T.SA_SCORE_INDEXER, q_idx=qi[2], k_idx=ki[2],
                                        idx_w=wi[2], scores=scores), reps)
    us_topk = timed(lambda: T.sa_topk(scores, k, idx_out=sel), reps)
    us_attend = timed(lambda: T.sa_sparse_decode(qs[2], ks[2], vs[2], sel, out=outs[2],
                                                 index_kind=T.SA_IDX_TOKEN_SHARED), reps)
    # the layer's own selection equals the calls' one
    layer(2, T.SA_LAYER_SPARSE)
    torch.cuda.synchronize()
    assert torch.equal(idx[2], sel), "sparse layer and its calls selected differently"
    dense_bytes = 2 * B * Hkv * N * d * 2
    score_bytes = B * N * Di * 2 + B * N * 4
    gather_bytes = 2 * B * Hkv * k * d * 2
    res = {
        "bench": "indexer1m: mixed 8-layer decode step", "unit": "us (HIP events)",
        "config": {"workload": "indexer1m: batch 1, 32/8 heads, d 128, bf16, 1048576 tokens, 8 layers "
                               "(2 dense, 6 sparse with a 4x64 shared indexer, top-2048)",
                   "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d, "ctx_len": N,
                   "k": k, "indexer_heads": H, "indexer_dim": Di, "modes": list(c.modes)},
        "mixed_step_us": round(us_mixed, 1), "all_dense_step_us": round(us_dense8, 1),
        "mixed_speedup_vs_all_dense": round(us_dense8 / us_mixed, 2),
        "dense_layer_us": round(us_dense, 1), "dense_layer_bytes": dense_bytes,
        "dense_layer_gbps": round(dense_bytes / us_dense / 1e3, 1),
        "sparse_layer_us": round(us_sparse, 1),
        "indexer_score_us": round(us_score, 1), "indexer_score_bytes": score_bytes,
        "indexer_score_gbps": round(score_bytes / us_score / 1e3, 1),
        "topk_us": round(us_topk, 1), "attend_us": round(us_attend, 1),
        "attend_bytes": gather_bytes, "attend_gbps": round(gather_bytes / us_attend / 1e3, 1),
        "data": "N(0,1) drawn on the device (seed %d)" % args.seed,
        "provenance": provenance()}
    for key in ("mixed_step_us", "all_dense_step_us", "mixed_speedup_vs_all_dense", "dense_layer_us",
                "dense_layer_gbps", "sparse_layer_us", "indexer_score_us", "indexer_score_gbps",
                "topk_us", "attend_us", "attend_gbps"):
        print("%28s  %s" % (key, res[key]))
    print(json.dumps(res), flush=True)


def block61k(args):
    """The block61k workload on the device: batch 8, 32/8 heads, d 128, bf16,
    61440 tokens = 480 blocks of 128, 24 blocks kept per (sequence, KV head),
    4 layers planned [SPARSE, REUSE 0, REUSE 0, REUSE 0].  Per call: the
    per-block key summaries (built once per cache, read K, write min/max),
    the block scores from the summaries, the top-24 of 480 and the gather-
    attend of the 3072 tokens of the kept blocks; then the 4-layer step
    against 4 dense layers.  Values are N(0,1) drawn on the device."""
    import torch
    import sa_synth as S
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    c = S.CONFIGS["block61k"]
    B, Hq, Hkv, d, N, bs, nblk, L = (c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.ctx_len,
                                     c.block_size, c.k, c.n_layers)
    nb = N // bs
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    log("block61k: drawing %d layers (%.1f GB of KV)" % (L, L * c.kv_bytes() / 1e9))

    def bf(shape):
        return torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(generator=gen)

    qs = [bf((B, Hq, d)) for _ in range(L)]
    ks = [bf((B, Hkv, N, d)) for _ in range(L)]
    vs = [bf((B, Hkv, N, d)) for _ in range(L)]
    kmin, kmax = T.sa_block_summarize(ks[0], bs, q_like=qs[0])
    scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, nblk), dtype=torch.int32, device=dev)
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
    largs = [T.layer_args(qs[l], ks[l], vs[l], T.SA_SCORE_BLOCK_MINMAX, nblk, kmin=kmin, kmax=kmax,
                          block_size=bs, out=outs[l])[0] for l in range(L)]
    modes = [T.SA_LAYER_DENSE if m == "dense" else T.SA_LAYER_SPARSE if m == "sparse" else
             T.SA_LAYER_REUSE for m in c.modes]
    T.sa_plan_validate(modes, list(c.src))
    ws = {m: T.WORKSPACES.get(dev, ("block61k", m), T.sa_layer_workspace_size(largs[0], m))
          for m in (T.SA_LAYER_DENSE, T.SA_LAYER_SPARSE, T.SA_LAYER_REUSE)}
    reps = max(3, min(args.steps, 10))

    def layer(l, m):
        T.sa_decode_layer(largs[l], m, None if m == T.SA_LAYER_DENSE else idx, dev, ws[m])

    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        layer(0, T.SA_LAYER_DENSE)  # queued ahead, so the host enqueues the rest in time
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    us_summ = timed(lambda: T.sa_block_summarize(ks[0], bs, q_like=qs[0], kmin=kmin, kmax=kmax), reps)
    us_score = timed(lambda: T.sa_score(qs[0], ks[0], T.SA_SCORE_BLOCK_MINMAX, kmin=kmin, kmax=kmax,
                                        block_size=bs, scores=scores), reps)
    us_topk = timed(lambda: T.sa_topk(scores, nblk, idx_out=idx), reps)
    us_attend = timed(lambda: T.sa_sparse_decode(qs[0], ks[0], vs[0], idx, out=outs[0],
                                                 index_kind=T.SA_IDX_BLOCK_PER_KV_HEAD,
                                                 block_size=bs), reps)
    us_sparse = timed(lambda: layer(0, T.SA_LAYER_SPARSE), reps)
    us_reuse = timed(lambda: layer(1, T.SA_LAYER_REUSE), reps)
    us_dense = timed(lambda: layer(0, T.SA_LAYER_DENSE), reps)
    us_plan = timed(lambda: [layer(l, modes[l]) for l in range(L)], reps)
    us_dense4 = timed(lambda: [layer(l, T.SA_LAYER_DENSE) for l in range(L)], reps)
    rows = B * Hkv
    summ_bytes = rows * N * d * 2 + 2 * rows * nb * d * 2
    score_bytes = 2 * rows * nb * d * 2 + B * Hq * d * 2 + rows * nb * 4
    topk_bytes = rows * nb * 4 + rows * nblk * 4
    attend_bytes = 2 * rows * nblk * bs * d * 2 + rows * nblk * 4 + 2 * B * Hq * d * 2 + B * Hq * d * 4
    dense_bytes = 2 * rows * N * d * 2

    def rate(nbytes, us):
        return {"us": round(us, 1), "bytes": nbytes, "gbps": round(nbytes / us / 1e3, 1),
                "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}

    res = {
        "bench": "block61k: block selection and reuse on the device", "unit": "us (HIP events)",
        "config": {"workload": "block61k: batch 8, 32/8 heads, d 128, bf16, 61440 tokens = 480 "
                               "blocks of 128, 24 blocks kept; 4 layers [SPARSE, REUSE x3]",
                   "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d, "ctx_len": N,
                   "block_size": bs, "blocks_kept": nblk, "modes": list(c.modes)},
        "block_summarize": rate(summ_bytes, us_summ),
        "block_score": rate(score_bytes, us_score),
        "block_topk": rate(topk_bytes, us_topk),
        "block_attend": rate(attend_bytes, us_attend),
        "sparse_layer_us": round(us_sparse, 1), "reuse_layer_us": round(us_reuse, 1),
        "dense_layer": rate(dense_bytes, us_dense),
        "plan_4_layers_us": round(us_plan, 1), "all_dense_4_layers_us": round(us_dense4, 1),
        "plan_speedup_vs_all_dense": round(us_dense4 / us_plan, 2),
        "data": "N(0,1) drawn on the device (seed %d)" % args.seed,
        "provenance": provenance()}
    for key in ("block_summarize", "block_score", "block_topk", "block_attend", "dense_layer"):
        print("%18s  %s" % (key, res[key]))
    for key in ("sparse_layer_us", "reuse_layer_us", "plan_4_layers_us", "all_dense_4_layers_us",
                "plan_speedup_vs_all_dense"):
        print("%18s  %s" % (key, res[key]))
    print(json.dumps(res), flush=True)


def hylra(args):
    """Layer-reuse policy on 8 layers of the llama32k shape.

    Queries and keys of layer l follow x_l = rho_l x_{l-1} + sqrt(1 - rho_l^2) z_l
    with the hylra32k schedule (a weakly correlated layer 4), drawn on the
    device (timings depend on the shapes and the plan, not on the values).
    Offline: every layer runs DENSE_SELECT, sa_index_overlap gives the
    overlap matrix, sa_plan_reuse the policy.  Then one 8-layer decode step is
    timed under each plan."""
    import torch
    import sa_synth as S
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    c = S.CONFIGS["hylra32k"]
    B, Hq, Hkv, d, N, k, L = c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.ctx_len, c.k, c.n_layers
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    log("hylra: drawing %d layers (%.1f GB of KV)" % (L, L * c.kv_bytes() / 1e9))
    qs, ks, vs = [], [], []
    xq = torch.randn((B, Hq, d), generator=gen, device=dev)
    xk = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev)
    for l in range(L):
        if l > 0:
            r = c.rho_sched[l]
            xq = r * xq + (1 - r * r) ** 0.5 * torch.randn(xq.shape, generator=gen, device=dev)
        qs.append(xq.to(torch.bfloat16).contiguous())
        kl = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev)
        for b in range(B):     # the fp32 latent chain one sequence at a time
            z = torch.randn((Hkv, N, d), generator=gen, device=dev)
            if l > 0:
                r = c.rho_sched[l]
                z = r * xk[b].float() + (1 - r * r) ** 0.5 * z
            xk[b] = z.to(torch.bfloat16)
            kl[b] = xk[b]
        ks.append(kl)
        vs.append(torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev).normal_(generator=gen))
    del xk
    torch.cuda.synchronize()
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
    largs = []
    for l in range(L):
        a, _, _ = T.layer_args(qs[l], ks[l], vs[l], T.SA_SCORE_EXACT, k, out=outs[l])
        largs.append(a)
    ws = {}
    for mode in (T.SA_LAYER_DENSE, T.SA_LAYER_SPARSE, T.SA_LAYER_REUSE, T.SA_LAYER_DENSE_SELECT):
        ws[mode] = T.WORKSPACES.get(dev, ("hylra", mode), T.sa_layer_workspace_size(largs[0], mode))
    idx = [torch.empty((B, Hkv, k), dtype=torch.int32, device=dev) for _ in range(L)]

    def run(modes, src):
        for l in range(L):
            m = modes[l]
            i = idx[src[l]] if m == T.SA_LAYER_REUSE else (None if m == T.SA_LAYER_DENSE else idx[l])
            T.sa_decode_layer(largs[l], m, i, dev, ws[m])

    # offline profiling: every layer full attention + its top-k, then overlaps
    run([T.SA_LAYER_DENSE_SELECT] * L, [-1] * L)
    M = np.zeros((L, L), dtype=np.int64)
    for i in range(L):
        for j in range(i + 1, L):
            M[i, j] = int(T.sa_index_overlap(idx[i], idx[j]).sum().item())
    total = B * Hkv * k
    ratio = M / total
    plans = {
        "all_dense": ([T.SA_LAYER_DENSE] * L, [-1] * L),
        "all_sparse_exact": ([T.SA_LAYER_SPARSE] * L, [-1] * L),
        "fixed_jump3": T.sa_plan_fixed_jump(L, 3),
        "hylra_dp": T.sa_plan_reuse(M, total, args.theta),
    }
    reps = max(3, min(args.steps, 20))
    res = {}
    for name, (modes, src) in plans.items():
        T.sa_plan_validate(modes, src)
        for _ in range(2):
            run(modes, src)
        torch.cuda.synchronize()
        # a long launch ahead of the timed region lets the host queue every
        # layer before the GPU reaches it
        T.sa_decode_layer(largs[0], T.SA_LAYER_DENSE, None, dev, ws[T.SA_LAYER_DENSE])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run(modes, src)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        reused = [ratio[src[l], l] for l in range(L) if modes[l] == T.SA_LAYER_REUSE]
        res[name] = {"modes": modes, "src": src, "us_per_step": round(us, 1),
                     "full_layers": sum(m in (T.SA_LAYER_DENSE, T.SA_LAYER_DENSE_SELECT)
                                        for m in modes),
                     "min_reused_overlap": round(min(reused), 4) if reused else None,
                     "mean_reused_overlap": round(float(np.mean(reused)), 4) if reused else None}
        log("hylra: %s %.1f us" % (name, us))
    # one layer per mode (layer 0; REUSE over layer 0's own set)
    per_layer = {}
    for name, m in (("dense", T.SA_LAYER_DENSE), ("dense_select", T.SA_LAYER_DENSE_SELECT),
                    ("sparse_exact", T.SA_LAYER_SPARSE), ("reuse", T.SA_LAYER_REUSE)):
        i = None if m == T.SA_LAYER_DENSE else idx[0]
        for _ in range(2):
            T.sa_decode_layer(largs[0], m, i, dev, ws[m])
        T.sa_decode_layer(largs[1], T.SA_LAYER_DENSE, None, dev, ws[T.SA_LAYER_DENSE])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            T.sa_decode_layer(largs[0], m, i, dev, ws[m])
        e1.record()
        torch.cuda.synchronize()
        per_layer[name] = round(e0.elapsed_time(e1) / reps * 1e3, 1)
    log("hylra: per layer %s" % per_layer)
    base = res["all_dense"]["us_per_step"]
    for r in res.values():
        r["speedup_vs_dense"] = round(base / r["us_per_step"], 3)
    print(json.dumps({
        "bench": "layer-reuse policy, 8-layer decode step", "unit": "us per 8-layer step (HIP events)",
        "config": {"workload": "hylra32k: llama32k shape x 8 layers, per-layer correlated q and K",
                   "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d, "ctx_len": N,
                   "k": k, "rho_sched": list(c.rho_sched), "theta": args.theta},
        "overlap_ratio": [[round(float(x), 4) for x in row] for row in ratio],
        "plans": res, "us_per_layer": per_layer,
        "data": "drawn on the device (torch generator, seed %d)" % args.seed,
        "provenance": provenance()}), flush=True)


def offload(args):
    """Index-guided offload on the block61k shape (batch 8, 32/8 heads, d 128,
    bf16, 61440 tokens = 480 blocks of 128, 24 blocks kept per row).

    Layer 0's cache is on the device; it selects blocks from min/max
    summaries.  Layers 1-3 keep their caches in pinned host memory and reuse
    layer 0's blocks: sa_gather_blocks fetches only those blocks, and dense
    decode over the gathered rows is their attention.  Values are drawn on
    the device; timings depend on the sizes only."""
    import torch
    import sa_synth as S
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    c = S.CONFIGS["block61k"]
    B, Hq, Hkv, d, N, bs, nblk = (c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.ctx_len,
                                  c.block_size, c.k)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    shape = (B, Hkv, N, d)
    log("offload: drawing 4 layers (%.1f GB of KV, 3 layers in pinned host memory)" % (
        4 * c.kv_bytes() / 1e9))
    qs = [torch.randn((B, Hq, d), generator=gen, device=dev).to(torch.bfloat16) for _ in range(4)]
    k0 = torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(generator=gen)
    v0 = torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(generator=gen)
    host = []
    for _ in range(3):
        kh = torch.empty(shape, dtype=torch.bfloat16, pin_memory=True)
        vh = torch.empty(shape, dtype=torch.bfloat16, pin_memory=True)
        for t in (kh, vh):
            t.copy_(torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(generator=gen))
        host.append((kh, vh))
    torch.cuda.synchronize()
    # layer 0: block selection on the device
    kmin, kmax = T.sa_block_summarize(k0, bs, q_like=qs[0])
    args0, out0, _ = T.layer_args(qs[0], k0, v0, T.SA_SCORE_BLOCK_MINMAX, nblk, kmin=kmin,
                                  kmax=kmax, block_size=bs)
    idx = torch.empty((B, Hkv, nblk), dtype=torch.int32, device=dev)
    T.sa_decode_layer(args0, T.SA_LAYER_SPARSE, idx, dev)
    torch.cuda.synchronize()
    sel_shape = (B, Hkv, nblk * bs, d)
    stage = [(torch.empty(sel_shape, dtype=torch.bfloat16, device=dev),
              torch.empty(sel_shape, dtype=torch.bfloat16, device=dev)) for _ in range(2)]
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(3)]
    reps = max(3, min(args.steps, 10))

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    kh, vh = host[0]
    us_gather = timed(lambda: T.sa_gather_blocks(kh, vh, idx, bs, *stage[0]), reps)
    us_attend = timed(lambda: T.sa_dense_decode(qs[1], *stage[0], out=outs[0]), reps)
    full_k = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    full_v = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    us_full = timed(lambda: (full_k.copy_(kh, non_blocking=True),
                             full_v.copy_(vh, non_blocking=True)), 2)
    # reuse layers 1-3: layer l attends while layer l+1's blocks are fetched
    # on a second stream (default priority)
    side = torch.cuda.Stream(device=dev)
    main_s = torch.cuda.current_stream(dev)

    def pipeline():
        done = [torch.cuda.Event() for _ in range(3)]
        with torch.cuda.stream(side):
            T.sa_gather_blocks(*host[0], idx, bs, *stage[0])
            done[0].record(side)
        for l in range(3):
            if l + 1 < 3:
                with torch.cuda.stream(side):
                    if l >= 1:
                        side.wait_event(used[l - 1])
                    T.sa_gather_blocks(*host[l + 1], idx, bs, *stage[(l + 1) % 2])
                    done[l + 1].record(side)
            main_s.wait_event(done[l])
            T.sa_dense_decode(qs[l + 1], *stage[l % 2], out=outs[l])
            used[l].record(main_s)

    used = [torch.cuda.Event() for _ in range(3)]
    us_pipe = timed(pipeline, reps)
    sel_bytes = 2 * B * Hkv * nblk * bs * d * 2
    full_bytes = 2 * B * Hkv * N * d * 2
    res = {
        "bench": "index-guided offload (HyLRA section 2.4)", "unit": "us (HIP events)",
        "config": {"workload": "block61k: batch 8, 32/8 heads, d 128, bf16, 61440 tokens, "
                               "24 of 480 blocks of 128 per row; layers 1-3 in pinned host memory",
                   "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d, "ctx_len": N,
                   "block_size": bs, "blocks_kept": nblk},
        "gather_selected_us": round(us_gather, 1), "gather_bytes": sel_bytes,
        "gather_host_link_gbps": round(sel_bytes / us_gather / 1e3, 1),
        "attend_gathered_us": round(us_attend, 1),
        "full_layer_copy_us": round(us_full, 1), "full_layer_bytes": full_bytes,
        "full_copy_host_link_gbps": round(full_bytes / us_full / 1e3, 1),
        "per_layer_speedup_vs_full_copy": round(us_full / (us_gather + us_attend), 2),
        "reuse_pipeline_3_layers_us": round(us_pipe, 1),
        "data": "drawn on the device (torch generator, seed %d)" % args.seed,
        "provenance": provenance()}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.summarize:
        print(summarize(args.summarize)[0])
        return
    if args.traffic:
        print(traffic_report(*args.traffic))
        return
    if args.gpus == 1 and args.sweep:
        sweep(args)
        return
    if args.gpus == 1 and args.block61k:
        block61k(args)
        return
    if args.gpus == 1 and args.indexer1m:
        indexer1m(args)
        return
    if args.gpus == 1 and args.nscale:
        nscale(args)
        return
    if args.gpus == 1 and args.hylra:
        hylra(args)
        return
    if args.gpus == 1 and args.offload:
        offload(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.profile:
        # plain launches (no graph capture) under the profiler
        args.steps, args.warmup, args.cpu_seconds, args.dense_steps = 20, 5, 0.0, 0
        args.cold_iters, args.eager, args.stream_gib = 0, True, 0

    import torch
    import sa_synth as S
    import top_sparse_decode_sa_amd as T

    T.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    w = S.Workload(args.workload, args.seed)
    c = w.cfg
    assert c.planting == "direction" and c.block_size == 0, "bench workload must be exact top-k"
    log("bench: generating %s (%.2f GB of KV) ..." % (c.name, c.kv_bytes() / 1e9))
    t0 = time.perf_counter()
    k_host, v_host = w.k(), w.v()
    q_host = [w.q(qvar=i) for i in range(N_QVAR)]
    log("bench: generated in %.1f s; uploading" % (time.perf_counter() - t0))

    def up(x):
        t = torch.from_numpy(x)
        return (t.view(torch.bfloat16) if t.dtype == torch.uint16 else t).to(dev)

    kd, vd = up(k_host), up(v_host)
    # R replicas of the cache (device copies), rotated with the queries
    n_rep = max(1, args.kv_replicas)
    kds = [kd] + [kd.clone() for _ in range(n_rep - 1)]
    vds = [vd] + [vd.clone() for _ in range(n_rep - 1)]
    qd = [up(q) for q in q_host]
    rows = c.batch * c.n_kv_heads
    scores = torch.empty((c.batch, c.n_kv_heads, c.ctx_len), dtype=torch.float32, device=dev)
    idx = torch.empty((c.batch, c.n_kv_heads, c.k), dtype=torch.int32, device=dev)
    out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i, ev=None):
        # exact selection (fused scoring + part top-k, then the merge), then
        # the gather-attend
        q = qd[i % N_QVAR]
        kr, vr = kds[i % n_rep], vds[i % n_rep]
        if ev is not None:
            ev[0].record()
        T.sa_select(q, kr, c.k, idx_out=idx)
        if ev is not None:
            ev[1].record()
        T.sa_sparse_decode(q, kr, vr, idx, out=out)
        if ev is not None:
            ev[2].record()

    log("bench: warmup %d steps" % args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed steps: each step captured once per query variant as a HIP
    # graph (the three launches of one decode step), replayed in turn
    graphs = []
    n_graph = N_QVAR * n_rep // math.gcd(N_QVAR, n_rep)
    if not args.eager:
        for v in range(n_graph):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(v)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % n_graph].replay()
        torch.cuda.synchronize()
        # a replayed step selects and attends exactly as the eager one
        graphs[0].replay()
        g_idx, g_out = idx.clone(), out.clone()
        step(0)
        torch.cuda.synchronize()
        assert torch.equal(g_idx, idx) and torch.equal(g_out, out), "graph replay differs from eager"

    log("bench: timing %d steps (%s)" % (args.steps, "eager" if args.eager else "graph replay"))
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        if args.eager:
            step(i)
        else:
            graphs[i % n_graph].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = wall * 1e3 / args.steps

    # per-kernel durations: eager steps with HIP events between the calls, on
    # the launch stream (a separate pass, so the events do not slow the
    # timed steps)
    n_ev = min(args.steps, 100)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    torch.cuda.synchronize()
    t_ev = time.perf_counter()
    for i in range(n_ev):
        step(i, events[i])
    torch.cuda.synchronize()
    ms_step_eager = (time.perf_counter() - t_ev) * 1e3 / n_ev
    ms_select = sum(e[0].elapsed_time(e[1]) for e in events) / n_ev
    ms_attend = sum(e[1].elapsed_time(e[2]) for e in events) / n_ev

    # the unfused selection on the same inputs, for comparison: every score
    # written by sa_score, then sa_topk over them (same index list)
    n_un = min(n_ev, 20)
    ev_un = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_un)]
    for i in range(2):
        T.sa_score(qd[i % N_QVAR], kd, T.SA_SCORE_EXACT, scores=scores)
        T.sa_topk(scores, c.k, idx_out=idx)
    torch.cuda.synchronize()
    for i in range(n_un):
        ev_un[i][0].record()
        T.sa_score(qd[i % N_QVAR], kd, T.SA_SCORE_EXACT, scores=scores)
        ev_un[i][1].record()
        T.sa_topk(scores, c.k, idx_out=idx)
        ev_un[i][2].record()
    torch.cuda.synchronize()
    ms_score = sum(e[0].elapsed_time(e[1]) for e in ev_un) / n_un
    ms_topk = sum(e[1].elapsed_time(e[2]) for e in ev_un) / n_un

    if args.profile:
        # plain device-to-device copies of known size: the byte counters of
        # these launches calibrate the counters of the kernels above
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # dense decode over the same cache (comparison for the sparse/dense ratio)
    ms_dense = None
    if args.dense_steps > 0:
        dout = torch.empty_like(out)
        for i in range(3):
            T.sa_dense_decode(qd[i % N_QVAR], kd, vd, out=dout)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.dense_steps):
            T.sa_dense_decode(qd[i % N_QVAR], kd, vd, out=dout)
        e1.record()
        torch.cuda.synchronize()
        ms_dense = e0.elapsed_time(e1) / args.dense_steps

    # the device's streaming read rate (sa_stream_read over 8 GiB): the
    # reference the rates above are also read against
    stream = None
    if args.stream_gib > 0:
        nbytes_s = args.stream_gib << 30
        buf = torch.empty(nbytes_s, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(2):
            T.sa_stream_read(buf, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            T.sa_stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        us_s = e0.elapsed_time(e1) / 5 * 1e3
        stream = {"bytes": nbytes_s, "us": round(us_s, 1), "gbps": round(nbytes_s / us_s / 1e3, 1),
                  "frac": round(nbytes_s / us_s / 1e3 / HBM_PEAK_GBPS, 4)}
        del buf, sink
        torch.cuda.empty_cache()

    # cache-cold gather-attend: before each launch a 1 GiB read evicts L2 and
    # the 256 MB last-level cache, as other layers' traffic would between
    # decode steps; beside it, the same kernel over the same number of bytes
    # read contiguously (a dense decode of the first k tokens of every row),
    # the cold-read floor at this size
    cold = None
    if args.cold_iters > 0:
        flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        kpre, vpre = kd[:, :, :c.k], vd[:, :, :c.k]
        cout = torch.empty_like(out)
        times = {"sparse": [], "contig": []}
        for i in range(args.cold_iters + 2):
            for name in ("sparse", "contig"):
                flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                if name == "sparse":
                    T.sa_sparse_decode(qd[0], kd, vd, idx, out=cout)
                else:
                    T.sa_dense_decode(qd[0], kpre, vpre, out=cout)
                e1.record()
                torch.cuda.synchronize()
                if i >= 2:
                    times[name].append(e0.elapsed_time(e1))
        del flush
        cold = {name: float(np.median(v)) for name, v in times.items()}

    nbytes = step_bytes(c)
    step_total = nbytes["select"] + nbytes["sparse_attend"]
    gbps = step_total / (ms_step * 1e-3) / 1e9

    def kern(name, ms):
        if ms is None:
            return None
        g = nbytes[name] / (ms * 1e-3) / 1e9
        return {"bytes": nbytes[name], "us": round(ms * 1e3, 3), "gbps": round(g, 1),
                "frac": round(g / HBM_PEAK_GBPS, 4)}

    kernels = {"select": kern("select", ms_select),
               "sparse_attend": kern("sparse_attend", ms_attend),
               "score_exact": kern("score_exact", ms_score), "topk": kern("topk", ms_topk),
               "dense_decode": kern("dense_decode", ms_dense)}
    if cold:
        kernels["sparse_attend_cold"] = kern("sparse_attend", cold["sparse"])
        kernels["contiguous_same_bytes_cold"] = kern("sparse_attend", cold["contig"])
    # dominant kernel of the step: the one with the largest share of its time
    dom = max(["select", "sparse_attend"], key=lambda n: kernels[n]["us"])
    roof = {"bound": "hbm", "achieved": kernels[dom]["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": kernels[dom]["frac"],
            "traffic": read_traffic(dom), "kernel": dom,
            "bytes_per_launch": nbytes[dom]}
    if stream:
        roof["frac_of_stream_read"] = round(kernels[dom]["gbps"] / stream["gbps"], 4)

    cpu = None
    if args.cpu_seconds > 0:
        log("bench: oracle cpu baseline (bounded to %.0f s)" % args.cpu_seconds)
        step_s, done, total = cpu_baseline(w, q_host, k_host, v_host, args.cpu_seconds)
        cpu = {"value": round(step_total / step_s / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "steps_per_s": round(1.0 / step_s, 4),
               "sample": "fp64 numpy oracle, one thread: score+top-k+attend of %d of the %d "
                         "(sequence, KV head) rows of one step, scaled by %d/%d" % (
                             done, total, total, done)}
        cpu.update(host_cpu())

    line = {
        "metric": "sparse-decode attn: achieved HBM GB/s (% of peak) + decode steps/s at 50x",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "steps_per_s": round(1e3 / ms_step, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "timing": "eager launches" if args.eager else "each step a replayed HIP graph (3 launches)",
        "step": "sa_select (fused exact scoring + part top-k, merge) -> sa_sparse_decode",
        "ms_per_step_eager_with_events": round(ms_step_eager, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; planted heavy keys)",
        "config": {"workload": "llama3.1-8b-shaped decode, exact top-k at 50x sparsity",
                   "batch": c.batch, "n_q_heads": c.n_q_heads, "n_kv_heads": c.n_kv_heads,
                   "head_dim": c.head_dim, "ctx_len": c.ctx_len, "k": c.k,
                   "kv_dtype": c.dtype, "kv_replicas": n_rep, "parallelism": "single GPU"},
        "roofline": roof,
        "kernels": kernels,
        "sparse_over_dense_speedup": (round(ms_dense / ms_attend, 2) if ms_dense else None),
        "stream_read": stream,
        "value_frac_of_stream_read": (round(gbps / stream["gbps"], 4) if stream else None),
        "cpu_baseline": cpu,
        "provenance": provenance(clocks=not args.profile),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
