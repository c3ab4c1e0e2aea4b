"""Benchmark of the top-k sparse decode attention path on one MI355X.

Workload (default): the Llama-3.1-8B-shaped decode step -- batch 16, 32 query
/ 8 KV heads, head_dim 128, bf16 KV cache of 32768 tokens per sequence, exact
top-k per (sequence, KV head) at 50x sparsity (k = 655).  One step is one pass
of the whole hot path through the C ABI, the SPARSE layer call:
    sa_decode_layer(SPARSE) = exact scoring fused with a per-part top-k, then
    the merge of the parts' candidates and the gather-attend in one launch;
the same step as two calls (sa_select -> sa_sparse_decode, the same index list
and output) is timed beside it.
Queries rotate over 8 pre-generated variants and the steps over 8 device
copies of the cache (2.15 GB each, all resident in HBM before timing starts;
--kv-replicas), so consecutive steps select different tokens and no step
finds the previous step's rows in cache.

Timing: W untimed warmup steps, then K timed steps bracketed by
torch.cuda.synchronize().  Each step is captured once per (query variant,
cache copy) as a HIP graph of its launches and replayed (a serving
loop's form; --eager times plain launches instead); the bench checks that a
replay selects and attends exactly as an eager step.

Prints ONE JSON line.  `value` is the gather-attend's achieved HBM bandwidth
(its algorithmic bytes, 43.65 MB per call, over its time per call): each
(query variant, cache copy) pair's index set is selected once, the 8
sa_sparse_decode calls over the 8 copies are captured back to back in one
HIP graph, and its replays are timed with HIP events on the launch stream
(consecutive calls read different copies, 8 x 43.65 MB exceeding the 256 MB
last-level cache).  `roofline` is that kernel against the 8 TB/s peak;
`ms_per_step` / `steps_per_s` are the K timed full decode steps (selection +
gather-attend) and `step` their bandwidth; `kernels` holds per-call times:
the same attend's reads alone (sa_gather_read: the same plan, index and row
loads without the arithmetic, timed the same way; `roofline.frac_of_gather_read`
is its time over the attend's), the same attend timed inside eager steps,
the selection, the unfused
selection (sa_score then sa_topk) and a dense decode for comparison, and two
cache-cold single launches after a 1 GiB read -- the gather-attend and
sa_stream_read over the same number of bytes (the floor for one launch of
that size).  `stream_read` is sa_stream_read over 8 GiB.  `cpu_baseline`
times the CPU oracle's selected-set attention (and its full step) on whole
rows of one step, scaled to a step.

Other modes (each prints its own JSON line): --workload block61k |
indexer1m | batch128k (those workloads on their seeded inputs, with an
all-core oracle baseline; --block61k and --indexer1m are aliases), --sweep
(full step with four selection front ends against dense decode at 2x-500x
on the llama32k and batch128k shapes), --hylra (layer-reuse plans over 8
layers), --offload (selected blocks fetched from a pinned host cache),
--nscale (32K-128K tokens at fixed k), --perhead (per-query-head index
sets); --profile (a short run for rocprofv3), --traffic and --summarize
(reports from its results).
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
    p.add_argument("--workload", default="llama32k",
                   choices=["llama32k", "block61k", "batch128k", "indexer1m"],
                   help="llama32k: the default line; the others time that workload on its seeded "
                        "inputs and print one JSON line of their own (attend GB/s, step rate, "
                        "kernels, dense comparison, an all-core oracle cpu_baseline)")
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
    p.add_argument("--perhead", action="store_true",
                   help="per-query-head index sets on the llama32k workload: each query head "
                        "selects its own top-655 and attends over it ([B, Hq, k]); the cold "
                        "gather-attend, the step, the SPARSE layer call, the per-KV-head step "
                        "and dense decode; one JSON line")
    p.add_argument("--indexer1m", action="store_true", help="same as --workload indexer1m")
    p.add_argument("--block61k", action="store_true", help="same as --workload block61k")
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
    "sparse_attend": (["attend_pairs_kernel"], ["top_sparse_decode_sa_amd/csrc/attend.hip",
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
    # launches of the method's kernels split by the kernel that ran just
    # before each (e.g. a gather-attend inside a step follows the selection,
    # one of a back-to-back series follows another gather-attend)
    seq = db.execute("select name, start, end from kernels order by start").fetchall()
    by_prev = {}
    for (pname, _, _), (name, st, en) in zip(seq, seq[1:]):
        if "sa::" in name:
            by_prev.setdefault((name, pname), []).append(en - st)
    if by_prev:
        lines.append("")
        lines.append("%-58s %-40s %6s %10s %10s" % ("kernel", "after", "calls", "avg_us",
                                                    "median_us"))
        for (name, pname), d in sorted(by_prev.items(), key=lambda kv: (kv[0][0], -len(kv[1]))):
            d = np.asarray(d, dtype=np.float64)
            lines.append("%-58s %-40s %6d %10.2f %10.2f" % (name[:58], pname[:40], len(d),
                                                            d.mean() / 1e3, np.median(d) / 1e3))
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


def pmc_copy_kib(db_path, counter):
    """The counter's value for the 1 GiB calibration copies: the mean over the
    copy dispatches within half of the largest one (the cache copies and the
    calibration copies move 1 GiB each; smaller copies of outputs are left
    out)."""
    import sqlite3
    db = sqlite3.connect(db_path)
    vals = [v for (v,) in db.execute(
        "select value from counters_collection where counter_name = ? and "
        "kernel_name like '%copyBuffer%'", (counter,)).fetchall()]
    if not vals:
        raise SystemExit("no calibration copy in %s" % db_path)
    big = [v for v in vals if v >= 0.5 * max(vals)]
    return sum(big) / len(big), len(big)


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
    fk_copy, n_copy = pmc_copy_kib(fetch_db, "FETCH_SIZE")
    wk_copy, _ = pmc_copy_kib(write_db, "WRITE_SIZE")
    ff = COPY_BYTES / (fk_copy * 1024.0)
    wf = COPY_BYTES / (wk_copy * 1024.0)
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
             "#   rocprofv3 --pmc FETCH_SIZE -d %s -o %s -- python3 bench.py --profile"
             % db_dir_name(fetch_db),
             "#   rocprofv3 --pmc WRITE_SIZE -d %s -o %s -- python3 bench.py --profile"
             % db_dir_name(write_db),
             "#   python bench.py --traffic %s %s" % (fetch_db, write_db),
             "# bench.py --profile runs three 1 GiB device-to-device copies (and 14 more make the",
             "# cache copies) that read and write exactly 1073741824 bytes each; factor =",
             "# 1073741824 / (mean counter KiB of those copies * 1024); smaller copies of outputs",
             "# are left out of the mean",
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


def cpu_baseline(w, q_host, k_host, v_host, idx_host, seconds):
    """Time the oracle, one BLAS thread, on whole (sequence, KV head) rows of
    one step until `seconds` elapse: its selected-set attention over the
    GPU's index set of the row (the headline's unit) and its full step
    (exact scores, top-k, attention).  Returns (seconds of attention per
    step, seconds of the full step per step, rows timed, rows)."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    c = w.cfg
    scale = O.default_scale(c.head_dim)
    rows = c.batch * c.n_kv_heads
    rows_done = 0
    t_att = t_step = 0.0
    with threadpool_limits(limits=1):
        qf = O.widen(q_host[0])
        t_all = time.perf_counter()
        for row in range(rows):
            b, r = divmod(row, c.n_kv_heads)
            qg = qf[b, r * c.group:(r + 1) * c.group]
            t0 = time.perf_counter()
            kf = O.widen(k_host[b, r])
            vf = O.widen(v_host[b, r])
            t1 = time.perf_counter()
            O.attend(qg, kf, vf, idx_host[b, r], scale)
            t2 = time.perf_counter()
            s = O.scores_exact(qg, kf, scale)
            sel = O.topk(s, c.k)
            O.attend(qg, kf, vf, sel, scale)
            t3 = time.perf_counter()
            # the rows' widening to fp64 is part of both
            t_att += (t1 - t0) + (t2 - t1)
            t_step += (t1 - t0) + (t3 - t2)
            rows_done += 1
            if time.perf_counter() - t_all >= seconds:
                break
    return t_att * rows / rows_done, t_step * rows / rows_done, rows_done, rows


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
    Both shapes use their seeded workloads (batch128k: 68.7 GB of K/V, the
    262 planted keys of each row).  attend_us is the median cache-cold
    gather-attend launch (a 1 GiB read before each): timed back to back, the
    batch128k gather (at most 137 MB) would find its rows in the 256 MB
    last-level cache.  The step columns read every key (or indexer key) row
    first, which evicts the gathered rows."""
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
        w = S.Workload(shape, args.seed)
        kd, vd, _, _ = upload_kv(w, 0, dev)
        q = torch.from_numpy(w.q()).view(torch.bfloat16).to(dev)
        data = "seeded %s workload (planted heavy keys)" % shape
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
            row["attend_us"] = round(_cold_us({"a": attend}, reps, dev)["a"], 1)
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
    value, so both grow linearly.  The seeded llama32k workload at each
    context length (1 % planted heavy keys), generated on the host."""
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

    import dataclasses
    import sa_synth as S

    for N in NSCALE_N:
        log("nscale: N=%d" % N)
        cN = dataclasses.replace(S.CONFIGS["llama32k"], ctx_len=N, k=k,
                                 n_planted=int(0.01 * N))
        w = S.Workload(cN, args.seed)
        kd, vd, _, _ = upload_kv(w, 0, dev)
        q = torch.from_numpy(w.q()).view(torch.bfloat16).to(dev)
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
                      "rows": rows, "data": "synthetic: the seeded llama32k workload at each "
                                            "context length (seed %d)" % args.seed,
                      "provenance": provenance()}), flush=True)


# ---------------------------------------------------------------------------
# The three other workloads on their seeded inputs (--workload NAME)
# ---------------------------------------------------------------------------

CPU_SHARE = 16   # oracle worker processes at most: one GPU's share of the host's cores


def cpu_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(CPU_SHARE, n))


def _oracle_prepare(cfg, seed, task, shm):
    """Generate (untimed) the inputs of one unit of the oracle's work and
    return a function that runs the unit and gives its seconds per part."""
    import oracle as O
    import sa_synth as S

    w = S.Workload(cfg, seed)
    c = w.cfg
    G, scale = c.group, O.default_scale(c.head_dim)
    clock = time.perf_counter
    kind = task[0]
    if kind == "row":          # one (sequence, KV head) row of an exact top-k layer
        _, b, r = task
        q = w.q(0, batch=(b, b + 1))[0, r * G:(r + 1) * G]
        k, v = w.k_row(0, b, r), w.v_row(0, b, r)

        def run():
            t0 = clock()
            qg, kf = O.widen(q), O.widen(k)
            t1 = clock()
            sel = O.topk(O.scores_exact(qg, kf, scale), c.k)
            t2 = clock()
            O.attend(qg, O.widen(k[sel]), O.widen(v[sel]), np.arange(c.k), scale)
            t3 = clock()
            O.dense(qg, kf, O.widen(v), scale)
            t4 = clock()
            return {"select": t2 - t0, "attend": t3 - t2, "dense": (t1 - t0) + (t4 - t3)}
        return run
    if kind == "block_row":    # one row of the 4-layer block plan
        _, b, r = task
        qs = [w.q(l, batch=(b, b + 1))[0, r * G:(r + 1) * G] for l in range(c.n_layers)]
        ks = [w.k_row(l, b, r) for l in range(c.n_layers)]
        vs = [w.v_row(l, b, r) for l in range(c.n_layers)]

        def run():
            t0 = clock()
            kf = O.widen(ks[0])
            kmin, kmax = O.block_summaries(kf, c.block_size)
            t1 = clock()
            q0 = O.widen(qs[0])
            blocks = O.topk(O.scores_block(q0, kmin, kmax), c.k)
            toks = O.block_tokens(blocks, c.block_size, c.ctx_len)
            t2 = clock()
            for l in range(c.n_layers):   # layer 0 SPARSE, layers 1-3 REUSE its blocks
                O.attend(O.widen(qs[l]), O.widen(ks[l][toks]), O.widen(vs[l][toks]),
                         np.arange(len(toks)), scale)
            t3 = clock()
            O.dense(q0, kf, O.widen(vs[0]), scale)
            t4 = clock()
            return {"summaries": t1 - t0, "select": t2 - t1, "attend": t3 - t2,
                    "dense": (t4 - t3) + (t1 - t0)}
        return run
    if kind == "dense_row":    # one row of a DENSE layer of the 1M-token plan
        _, layer, r = task
        q = w.q(layer)[0, r * G:(r + 1) * G]
        k, v = w.k_row(layer, 0, r), w.v_row(layer, 0, r)

        def run():
            t0 = clock()
            O.dense(O.widen(q), O.widen(k), O.widen(v), scale)
            return {"dense": clock() - t0}
        return run
    if kind == "indexer_layer":   # one SPARSE layer of the 1M-token plan (all 8 KV heads)
        _, layer = task
        z = np.load(os.path.join(shm, "layer%d.npz" % layer))
        qi, ki, wi, q = z["qi"], z["ki"], z["wi"], z["q"]

        def run():
            t0 = clock()
            sel = O.topk(O.scores_indexer(O.widen(qi[0]), O.widen(ki[0]), wi.astype(np.float64)),
                         c.k)
            t1 = clock()
            # the selected rows are drawn from the generator's counters (untimed)
            rows = [(w.kv_tokens("k", layer, 0, r, sel), w.kv_tokens("v", layer, 0, r, sel))
                    for r in range(c.n_kv_heads)]
            t2 = clock()
            for r, (kr, vr) in enumerate(rows):
                O.attend(O.widen(q[0, r * G:(r + 1) * G]), O.widen(kr), O.widen(vr),
                         np.arange(c.k), scale)
            t3 = clock()
            return {"select": t1 - t0, "attend": t3 - t2}
        return run
    raise ValueError(kind)


def _oracle_worker(cfg, seed, tasks, shm, barrier, results):
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        runs = [_oracle_prepare(cfg, seed, t, shm) for t in tasks]
        barrier.wait()
        out = [fn() for fn in runs]
    results.put(out)


def oracle_pool(cfg, seed, task_lists, shm=None):
    """Run the oracle's units in len(task_lists) worker processes, one BLAS /
    OpenMP thread each: every worker generates its inputs, all start the
    timed work together (a barrier), and each reports its units' seconds.
    Returns (per-part makespan: the largest per-worker sum, units done)."""
    import multiprocessing as mp

    ctx = mp.get_context("spawn")
    n = len(task_lists)
    barrier, results = ctx.Barrier(n), ctx.Queue()
    saved = {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS")}
    os.environ.update({v: "1" for v in saved})
    import queue

    procs = []
    try:
        procs = [ctx.Process(target=_oracle_worker, args=(cfg, seed, tl, shm, barrier, results))
                 for tl in task_lists]
        for p in procs:
            p.start()
        got = []
        while len(got) < len(procs):
            try:
                got.append(results.get(timeout=5.0))
            except queue.Empty:
                # a worker that died (out of memory, an exception) never reports
                dead = [p.exitcode for p in procs if p.exitcode not in (None, 0)]
                if dead:
                    barrier.abort()
                    raise RuntimeError("oracle worker failed (exit codes %s)" % dead)
        for p in procs:
            p.join()
    finally:
        for p in procs:
            if p.is_alive():
                p.terminate()
                p.join()
        for v, x in saved.items():
            if x is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = x
    sums = [{} for _ in got]
    for acc, worker in zip(sums, got):
        for unit in worker:
            for part, sec in unit.items():
                acc[part] = acc.get(part, 0.0) + sec

    def span(*parts):
        return max(sum(acc.get(p_, 0.0) for p_ in parts) for acc in sums)
    return span, sum(len(worker) for worker in got)


def _spread(tasks, n):
    """Deal tasks to n workers in turn."""
    return [tasks[i::n] for i in range(n) if tasks[i::n]]


def config_cpu_baseline(name, seed, attend_bytes, shm=None, cfg=None, workers=None):
    """The oracle on the host: one thread on a stated subset, then all the
    workers over a larger sample, each scaled to one step of the workload
    `name` (cfg: the same workload at other sizes)."""
    import sa_synth as S

    c = S.CONFIGS[name] if cfg is None else cfg
    W = workers or cpu_workers()
    if name == "batch128k":
        rows = c.batch * c.n_kv_heads
        one = [("row", 0, r) for r in range(c.n_kv_heads)]
        per = max(1, 64 // W)
        sample = [("row", (i * 37) % c.batch, i % c.n_kv_heads) for i in range(W * per)]
        one_unit, all_unit = rows / len(one), rows / len(sample)
        what = ("exact scores, top-%d and selected-set attention of (sequence, KV head) rows; "
                "dense: full attention of the same rows" % c.k)
    elif name == "block61k":
        rows = c.batch * c.n_kv_heads
        one = [("block_row", 0, r) for r in range(c.n_kv_heads)]
        sample = [("block_row", b, r) for b in range(c.batch) for r in range(c.n_kv_heads)]
        one_unit, all_unit = rows / len(one), rows / len(sample)
        what = ("per row: block scores from the layer-0 summaries, top-%d blocks, attention over "
                "their tokens at all %d layers (SPARSE + REUSE); summaries (once per cache) and "
                "dense layer 0 apart" % (c.k, c.n_layers))
    else:
        one = [("dense_row", 0, 0), ("indexer_layer", 2)]
        sample = [("indexer_layer", l) for l in range(c.n_layers) if c.modes[l] == "sparse"] + \
                 [("dense_row", l, r) for l in range(c.n_layers) if c.modes[l] == "dense"
                  for r in range(c.n_kv_heads)]
        one_unit = all_unit = None
        what = ("the 8-layer plan: dense rows of layers 0-1, and for layers 2-7 the indexer "
                "scores of all 1048576 tokens, the top-%d and the attention of the 8 KV heads "
                "over it" % c.k)
    log("%s: oracle on one thread (%d units)" % (name, len(one)))
    t0 = time.perf_counter()
    span1, n1 = oracle_pool(c, seed, [one], shm)
    log("%s: oracle on %d workers (%d units)" % (name, W, len(sample)))
    spanW, nW = oracle_pool(c, seed, _spread(sample, W), shm)
    wall = time.perf_counter() - t0
    if name == "indexer1m":
        n_dense = sum(1 for m in c.modes if m == "dense") * c.n_kv_heads
        n_sparse = sum(1 for m in c.modes if m == "sparse")
        # one thread: one dense row and one sparse layer, scaled to the plan
        step1 = n_dense * span1("dense") + n_sparse * span1("select", "attend")
        att1 = n_sparse * span1("attend")
        # all workers: the whole plan's units, so no scaling
        stepW, attW = spanW("dense", "select", "attend"), spanW("attend")
        dense1 = denseW = None
    else:
        step1 = span1("select", "attend") * one_unit
        att1 = span1("attend") * one_unit
        dense1 = span1("dense") * one_unit
        stepW = spanW("select", "attend") * all_unit
        attW = spanW("attend") * all_unit
        denseW = spanW("dense") * all_unit
    cpu = {"value": round(attend_bytes / attW / 1e9, 4), "unit": "GB/s", "cores": W,
           "kind": "oracle", "steps_per_s": round(1.0 / stepW, 4),
           "sample": "fp64 numpy oracle on %d worker processes of one thread (%s), %d units, "
                     "scaled to one step; value: its selected-set attention's algorithmic bytes "
                     "per step over its attention time" % (W, what, nW),
           "one_thread": {"steps_per_s": round(1.0 / step1, 4),
                          "attend_gbps": round(attend_bytes / att1 / 1e9, 4),
                          "sample": "units %s, scaled to one step" % (one,)},
           "wall_s": round(wall, 1)}
    if dense1 is not None:
        cpu["dense_steps_per_s"] = round(1.0 / denseW, 4)
        cpu["one_thread"]["dense_steps_per_s"] = round(1.0 / dense1, 4)
    cpu.update(host_cpu())
    return cpu


def _ev_us(fn, n, warm=2):
    """Mean microseconds per call over n back-to-back calls (HIP events on
    the current stream)."""
    import torch

    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def _graph_us(fns, n):
    """Microseconds per call of the calls fns captured back to back in one
    HIP graph, replayed n times between HIP events."""
    import torch

    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    return _ev_us(g.replay, n, warm=3) / len(fns)


def _cold_us(fns, iters, dev):
    """Cache-cold single launches: before each, a 1 GiB read evicts L2 and the
    256 MB last-level cache.  Returns {name: median us} over `iters` rounds."""
    import torch

    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    times = {name: [] for name in fns}
    for i in range(iters + 2):
        for name, fn in fns.items():
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                times[name].append(e0.elapsed_time(e1) * 1e3)
    del flush
    return {name: float(np.median(v)) for name, v in times.items()}


def _rate(nbytes, us):
    if us is None:
        return None
    g = nbytes / us / 1e3
    return {"bytes": int(nbytes), "us": round(us, 3), "gbps": round(g, 1),
            "frac": round(g / HBM_PEAK_GBPS, 4)}


def _stream_floor(nbytes, dev):
    """sa_stream_read over nbytes (rounded down to 16 B) as a cold single launch."""
    import torch
    import top_sparse_decode_sa_amd as T

    sbuf = torch.empty(nbytes // 16 * 16, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    return sbuf, (lambda: T.sa_stream_read(sbuf, sink))


def upload_kv(w, layer, dev, chunk=4):
    """K and V of one layer of a seeded workload, generated on the host in
    batch slices of `chunk` sequences and copied into device memory; returns
    (k, v, generation seconds, upload seconds)."""
    import torch

    c = w.cfg
    gen_s = up_s = 0.0
    tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    kd = torch.empty((c.batch, c.n_kv_heads, c.ctx_len, c.head_dim), dtype=tdt, device=dev)
    vd = torch.empty_like(kd)
    for b0 in range(0, c.batch, chunk):
        b1 = min(c.batch, b0 + chunk)
        for which, dst in (("k", kd), ("v", vd)):
            t0 = time.perf_counter()
            host = w.k(layer, batch=(b0, b1)) if which == "k" else w.v(layer, batch=(b0, b1))
            t1 = time.perf_counter()
            t = torch.from_numpy(host)
            dst[b0:b1].copy_(t.view(torch.bfloat16) if t.dtype == torch.uint16 else t)
            torch.cuda.synchronize()
            gen_s += t1 - t0
            up_s += time.perf_counter() - t1
            del host, t
    return kd, vd, gen_s, up_s


def _line(name, c, args, value_kernel, timing, extra):
    """One JSON line of a seeded-workload run."""
    at = value_kernel
    line = {
        "metric": "sparse-decode attn: achieved HBM GB/s (% of peak) + decode steps/s",
        "value": at["gbps"], "unit": "GB/s", "hbm_frac": at["frac"], "attend_us": at["us"],
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "timing": timing,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: the seeded %s workload (counter-based generator; generation and "
                "upload untimed)" % name,
        "roofline": {"bound": "hbm", "achieved": at["gbps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": at["frac"], "traffic": None,
                     "kernel": "sparse_attend", "bytes_per_launch": at["bytes"]},
    }
    line.update(extra)
    line["provenance"] = provenance()
    return line


def bench_batch128k(args):
    """batch 128, 32/8 heads, d 128, bf16, 131072 tokens (68.7 GB of KV), exact
    top-262 per (sequence, KV head) at 500x, the 262 planted heavy keys of each
    row.  The step: sa_select then sa_sparse_decode.  The gather-attend
    (137.4 MB) fits the 256 MB last-level cache, so back-to-back repeats would
    be cache hits: `value` is the median cache-cold single launch after a
    1 GiB read, beside a cold sa_stream_read of the same byte count."""
    import sa_synth as S

    name = "batch128k"
    c = S.CONFIGS[name]
    att_bytes = step_bytes(c)["sparse_attend"]
    cpu = config_cpu_baseline(name, args.seed, att_bytes) if args.cpu_seconds > 0 else None

    import torch
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    w = S.Workload(name, args.seed)
    log("%s: generating %.1f GB of KV" % (name, c.kv_bytes() / 1e9))
    kd, vd, gen_s, up_s = upload_kv(w, 0, dev)
    qd = [torch.from_numpy(w.q(0, qvar=v)).view(torch.bfloat16).to(dev) for v in range(2)]
    idx = torch.empty((c.batch, c.n_kv_heads, c.k), dtype=torch.int32, device=dev)
    out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device=dev)
    n_steps, n_warm = max(3, min(args.steps, 20)), max(1, min(args.warmup, 3))

    def select(i=0):
        T.sa_select(qd[i % 2], kd, c.k, idx_out=idx)

    def attend(i=0):
        T.sa_sparse_decode(qd[i % 2], kd, vd, idx, out=out)

    for i in range(n_warm):
        select(i)
        attend(i)
    torch.cuda.synchronize()
    # the selection is the planted set of every row
    planted = np.stack([[w.planted(0, b, r) for r in range(c.n_kv_heads)] for b in range(c.batch)])
    assert np.array_equal(idx.cpu().numpy(), planted), "selection differs from the planted sets"
    assert T.sa_check_indices(qd[0], kd, idx).tolist() == [0, 0]
    log("%s: timing %d steps" % (name, n_steps))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_steps):
        ev[i][0].record()
        select(i)
        ev[i][1].record()
        attend(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / n_steps
    us_sel = sum(e[0].elapsed_time(e[1]) for e in ev) / n_steps * 1e3
    us_att_step = sum(e[1].elapsed_time(e[2]) for e in ev) / n_steps * 1e3
    sbuf, stream = _stream_floor(att_bytes, dev)
    cold = _cold_us({"attend": attend, "stream": stream}, max(5, args.cold_iters), dev)
    del sbuf
    dout = torch.empty_like(out)
    us_dense = _ev_us(lambda: T.sa_dense_decode(qd[0], kd, vd, out=dout), 3, warm=1)
    nb = step_bytes(c)
    att = _rate(att_bytes, cold["attend"])
    kernels = {"sparse_attend_cold": att,
               "stream_read_same_bytes_cold": _rate(att_bytes // 16 * 16, cold["stream"]),
               "sparse_attend_in_step": _rate(att_bytes, us_att_step),
               "select": _rate(nb["select"], us_sel),
               "dense_decode": _rate(nb["dense_decode"], us_dense)}
    line = _line(name, c, args, att,
                 "value: median of %d cache-cold single gather-attend launches (HIP events), "
                 "each after a 1 GiB read; steps: %d eager steps (select + gather-attend) after "
                 "%d warmup" % (max(5, args.cold_iters), n_steps, n_warm),
                 {"ms_per_step": round(ms_step, 4), "steps_per_s": round(1e3 / ms_step, 2),
                  "config": {"workload": "batch128k: large batch at 500x sparsity, exact top-k",
                             "batch": c.batch, "n_q_heads": c.n_q_heads,
                             "n_kv_heads": c.n_kv_heads, "head_dim": c.head_dim,
                             "ctx_len": c.ctx_len, "k": c.k, "kv_dtype": c.dtype,
                             "parallelism": "single GPU"},
                  "kernels": kernels,
                  "sparse_over_dense_speedup": round(us_dense / cold["attend"], 2),
                  "step_over_dense_speedup": round(us_dense / (ms_step * 1e3), 3),
                  "generation_s": round(gen_s, 1), "upload_s": round(up_s, 1),
                  "cpu_baseline": cpu})
    line["roofline"]["cold_frac_of_same_bytes_stream"] = round(cold["stream"] / cold["attend"], 4)
    print(json.dumps(line), flush=True)


def bench_perhead(args):
    """Per-query-head index sets on the llama32k workload (batch 16, 32/8
    heads, d 128, bf16, 32768 tokens, k = 655): every query head scores the
    cache with its own query (SA_SCORE_EXACT_PER_Q_HEAD), keeps its own top-655
    and attends over its own set (SA_IDX_TOKEN_PER_Q_HEAD, [B, Hq, k]); beside
    it the per-KV-head step on the same inputs and dense decode.  A query
    head's gather is 655 key and value rows, so one step gathers four times
    the per-KV-head bytes (171.7 MB), which fits the 256 MB last-level cache:
    `value` is the median cache-cold single launch after a 1 GiB read, beside
    a cold streaming read of the same byte count."""
    import sa_synth as S

    name = "llama32k"
    c = S.CONFIGS[name]
    import torch
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    w = S.Workload(name, args.seed)
    B, Hq, Hkv, d, k = c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.k
    log("perhead: generating %s (%.2f GB of KV)" % (name, c.kv_bytes() / 1e9))
    kd, vd, gen_s, up_s = upload_kv(w, 0, dev)
    qd = [torch.from_numpy(w.q(0, qvar=v)).view(torch.bfloat16).to(dev) for v in range(2)]
    idx_q = torch.empty((B, Hq, k), dtype=torch.int32, device=dev)
    idx_kv = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    n_steps, n_warm = max(3, min(args.steps, 20)), max(1, min(args.warmup, 3))

    def select(i=0):
        T.sa_select(qd[i % 2], kd, k, T.SA_SCORE_EXACT_PER_Q_HEAD, idx_out=idx_q)

    def attend(i=0):
        T.sa_sparse_decode(qd[i % 2], kd, vd, idx_q, index_kind=T.SA_IDX_TOKEN_PER_Q_HEAD, out=out)

    largs = [T.layer_args(qd[v], kd, vd, T.SA_SCORE_EXACT_PER_Q_HEAD, k, out=out)[0] for v in range(2)]
    lws = torch.empty(max(1, T.sa_layer_workspace_size(largs[0], T.SA_LAYER_SPARSE)),
                      dtype=torch.uint8, device=dev)

    def layer(i=0):
        T.sa_decode_layer(largs[i % 2], T.SA_LAYER_SPARSE, idx_q, dev, lws)

    def kv_step(i=0):
        T.sa_select(qd[i % 2], kd, k, idx_out=idx_kv)
        T.sa_sparse_decode(qd[i % 2], kd, vd, idx_kv, out=out)

    for i in range(n_warm):
        select(i)
        attend(i)
        layer(i)
        kv_step(i)
    torch.cuda.synchronize()
    # the layer call selects and attends exactly as the two calls
    select(0)
    attend(0)
    two_idx, two_out = idx_q.clone(), out.clone()
    layer(0)
    torch.cuda.synchronize()
    assert torch.equal(two_idx, idx_q) and torch.equal(two_out, out), "layer call differs"
    assert T.sa_check_indices(qd[0], kd, idx_q, index_kind=T.SA_IDX_TOKEN_PER_Q_HEAD).tolist() == [0, 0]
    log("perhead: timing %d steps" % n_steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_steps)]
    torch.cuda.synchronize()
    for i in range(n_steps):
        ev[i][0].record()
        select(i)
        ev[i][1].record()
        attend(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    us_sel = sum(e[0].elapsed_time(e[1]) for e in ev) / n_steps * 1e3
    us_att_step = sum(e[1].elapsed_time(e[2]) for e in ev) / n_steps * 1e3
    us_layer = _ev_us(lambda: layer(1), n_steps, warm=2)
    us_kv_step = _ev_us(lambda: kv_step(1), n_steps, warm=2)
    att_bytes = 2 * B * Hq * k * d * c.elt + B * Hq * k * 4 + B * Hq * d * (c.elt + 4)
    sbuf, stream = _stream_floor(att_bytes, dev)
    cold = _cold_us({"attend": attend, "stream": stream}, max(5, args.cold_iters), dev)
    del sbuf
    dout = torch.empty_like(out)
    us_dense = _ev_us(lambda: T.sa_dense_decode(qd[0], kd, vd, out=dout), 3, warm=1)
    nb = step_bytes(c)
    # the selection's algorithmic bytes: the keys read once (one scoring
    # pass serves a KV head's query heads), the queries, every query head's
    # scores written and read back by the top-k, the index lists written
    sel_bytes = (B * Hkv * c.ctx_len * d * c.elt + B * Hq * d * c.elt + 2 * B * Hq * c.ctx_len * 4
                 + B * Hq * k * 4)
    att = _rate(att_bytes, cold["attend"])
    kernels = {"sparse_attend_cold": att,
               "stream_read_same_bytes_cold": _rate(att_bytes // 16 * 16, cold["stream"]),
               "sparse_attend_in_step": _rate(att_bytes, us_att_step),
               "select": _rate(sel_bytes, us_sel),
               "dense_decode": _rate(nb["dense_decode"], us_dense)}
    cpu = None
    if args.cpu_seconds > 0:
        cpu = perhead_cpu_baseline(w, att_bytes, args.cpu_seconds)
    line = _line("llama32k", c, args, att,
                 "value: median of %d cache-cold single per-query-head gather-attend launches "
                 "(HIP events), each after a 1 GiB read; steps: %d eager steps (sa_select per "
                 "query head + gather-attend) after %d warmup; layer: the SPARSE layer call with "
                 "per-query-head scores, back to back" % (max(5, args.cold_iters), n_steps, n_warm),
                 {"ms_per_step": round((us_sel + us_att_step) / 1e3, 4),
                  "steps_per_s": round(1e6 / (us_sel + us_att_step), 1),
                  "config": {"workload": "llama32k with per-query-head index sets ([B, Hq, k])",
                             "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d,
                             "ctx_len": c.ctx_len, "k": k, "kv_dtype": c.dtype,
                             "parallelism": "single GPU"},
                  "kernels": kernels,
                  "layer_us": round(us_layer, 1),
                  "per_kv_head_step_us": round(us_kv_step, 1),
                  "sparse_over_dense_speedup": round(us_dense / cold["attend"], 2),
                  "layer_over_dense_speedup": round(us_dense / us_layer, 3),
                  "generation_s": round(gen_s, 1), "upload_s": round(up_s, 1),
                  "cpu_baseline": cpu})
    line["roofline"]["cold_frac_of_same_bytes_stream"] = round(cold["stream"] / cold["attend"], 4)
    print(json.dumps(line), flush=True)


def perhead_cpu_baseline(w, att_bytes, seconds):
    """The oracle, one BLAS thread, on whole query-head rows of one step until
    `seconds` elapse: each head's exact scores over the cache, its top-k and
    its attention over that set; scaled to the step's B * Hq rows."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    c = w.cfg
    scale = O.default_scale(c.head_dim)
    rows = c.batch * c.n_q_heads
    done = 0
    t_att = t_step = 0.0
    with threadpool_limits(limits=1):
        t_all = time.perf_counter()
        b_loaded = -1
        for row in range(rows):
            b, h = divmod(row, c.n_q_heads)
            if b != b_loaded:
                k_b, v_b = w.k(0, batch=(b, b + 1))[0], w.v(0, batch=(b, b + 1))[0]
                qf = O.widen(w.q(0, batch=(b, b + 1))[0])
                b_loaded = b
            t0 = time.perf_counter()
            kf = O.widen(k_b[h // c.group])
            vf = O.widen(v_b[h // c.group])
            qh = qf[h:h + 1]
            t1 = time.perf_counter()
            sel = O.topk(O.scores_exact(qh, kf, scale), c.k)
            t2 = time.perf_counter()
            O.attend(qh, kf, vf, sel, scale)
            t3 = time.perf_counter()
            t_att += (t1 - t0) + (t3 - t2)
            t_step += t3 - t0
            done += 1
            if time.perf_counter() - t_all >= seconds:
                break
    att_s, step_s = t_att * rows / done, t_step * rows / done
    cpu = {"value": round(att_bytes / att_s / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle", "steps_per_s": round(1.0 / step_s, 4),
           "attend_steps_per_s": round(1.0 / att_s, 4),
           "sample": "fp64 numpy oracle, one thread: %d of the %d query-head rows of one step "
                     "(exact scores, top-k, attention over the head's own set), scaled by %d/%d"
                     % (done, rows, rows, done)}
    cpu.update(host_cpu())
    return cpu


def bench_block61k(args):
    """batch 8, 32/8 heads, d 128, bf16, 61440 tokens = 480 blocks of 128, the
    top 24 blocks per (sequence, KV head) from per-block key min/max
    summaries, 4 layers planned [SPARSE, REUSE 0 x 3] over keys correlated
    0.9 from layer to layer.  `value`: the block gather-attend (3072 tokens a
    row, 100.9 MB a layer), the four layers' attends over their own caches
    back to back in a HIP graph (403 MB, more than the last-level cache)."""
    import sa_synth as S

    name = "block61k"
    c = S.CONFIGS[name]
    bs, L = c.block_size, c.n_layers
    rows, nb = c.batch * c.n_kv_heads, c.ctx_len // c.block_size
    att_bytes = (2 * rows * c.k * bs * c.head_dim * 2 + rows * c.k * 4 + c.batch * c.n_q_heads *
                 c.head_dim * (2 + 4))
    cpu = config_cpu_baseline(name, args.seed, att_bytes * L) if args.cpu_seconds > 0 else None

    import torch
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    w = S.Workload(name, args.seed)
    log("%s: generating %d layers (%.1f GB of KV)" % (name, L, L * c.kv_bytes() / 1e9))
    gen_s = up_s = 0.0
    qs, ks, vs = [], [], []
    for l in range(L):
        t0 = time.perf_counter()
        kh, vh, qh = w.k(l), w.v(l), w.q(l)
        t1 = time.perf_counter()
        for h, lst in ((kh, ks), (vh, vs), (qh, qs)):
            lst.append(torch.from_numpy(h).view(torch.bfloat16).to(dev))
        torch.cuda.synchronize()
        gen_s += t1 - t0
        up_s += time.perf_counter() - t1
        del kh, vh, qh
    kmin, kmax = T.sa_block_summarize(ks[0], bs, q_like=qs[0])
    scores = torch.empty((c.batch, c.n_kv_heads, nb), dtype=torch.float32, device=dev)
    idx = torch.empty((c.batch, c.n_kv_heads, c.k), dtype=torch.int32, device=dev)
    outs = [torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device=dev)
            for _ in range(L)]
    largs = [T.layer_args(qs[l], ks[l], vs[l], T.SA_SCORE_BLOCK_MINMAX, c.k, kmin=kmin, kmax=kmax,
                          block_size=bs, out=outs[l])[0] for l in range(L)]
    modes = [T.SA_LAYER_SPARSE if m == "sparse" else T.SA_LAYER_REUSE for m in c.modes]
    T.sa_plan_validate(modes, list(c.src))
    ws = {m: T.WORKSPACES.get(dev, (name, m), T.sa_layer_workspace_size(largs[0], m))
          for m in (T.SA_LAYER_DENSE, T.SA_LAYER_SPARSE, T.SA_LAYER_REUSE)}

    def layer(l, m):
        T.sa_decode_layer(largs[l], m, None if m == T.SA_LAYER_DENSE else idx, dev, ws[m])

    def plan():
        for l in range(L):
            layer(l, modes[l])

    n_steps, n_warm = max(3, min(args.steps, 50)), max(1, min(args.warmup, 5))
    for _ in range(n_warm):
        plan()
    torch.cuda.synchronize()
    assert T.sa_check_indices(qs[0], ks[0], idx, T.SA_IDX_BLOCK_PER_KV_HEAD, bs).tolist() == [0, 0]
    log("%s: timing %d 4-layer steps" % (name, n_steps))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(L + 1)] for _ in range(n_steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_steps):
        for l in range(L):
            ev[i][l].record()
            layer(l, modes[l])
        ev[i][L].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / n_steps
    us_layer = [sum(e[l].elapsed_time(e[l + 1]) for e in ev) / n_steps * 1e3 for l in range(L)]

    def attend(l):
        return lambda: T.sa_sparse_decode(qs[l], ks[l], vs[l], idx, out=outs[l],
                                          index_kind=T.SA_IDX_BLOCK_PER_KV_HEAD, block_size=bs)

    reps = max(10, min(args.steps, 50))
    us_att = _graph_us([attend(l) for l in range(L)], reps)
    us_summ = _ev_us(lambda: T.sa_block_summarize(ks[0], bs, q_like=qs[0], kmin=kmin, kmax=kmax), 5)
    us_score = _ev_us(lambda: T.sa_score(qs[0], ks[0], T.SA_SCORE_BLOCK_MINMAX, kmin=kmin,
                                         kmax=kmax, block_size=bs, scores=scores), reps)
    us_topk = _ev_us(lambda: T.sa_topk(scores, c.k, idx_out=idx), reps)
    sbuf, stream = _stream_floor(att_bytes, dev)
    cold = _cold_us({"attend": attend(0), "stream": stream,
                     "sparse_layer": lambda: layer(0, T.SA_LAYER_SPARSE)},
                    max(5, args.cold_iters), dev)
    del sbuf
    us_dense = _ev_us(lambda: layer(0, T.SA_LAYER_DENSE), 5)
    us_dense4 = _ev_us(lambda: [layer(l, T.SA_LAYER_DENSE) for l in range(L)], 3)
    summ_bytes = rows * c.ctx_len * c.head_dim * 2 + 2 * rows * nb * c.head_dim * 2
    score_bytes = 2 * rows * nb * c.head_dim * 2 + c.batch * c.n_q_heads * c.head_dim * 2 + rows * nb * 4
    topk_bytes = rows * nb * 4 + rows * c.k * 4
    dense_bytes = 2 * rows * c.ctx_len * c.head_dim * 2
    att = _rate(att_bytes, us_att)
    kernels = {"sparse_attend": att, "sparse_attend_cold": _rate(att_bytes, cold["attend"]),
               "stream_read_same_bytes_cold": _rate(att_bytes // 16 * 16, cold["stream"]),
               "block_summarize": _rate(summ_bytes, us_summ),
               "block_score": _rate(score_bytes, us_score),
               "block_topk": _rate(topk_bytes, us_topk),
               "dense_layer": _rate(dense_bytes, us_dense)}
    line = _line(name, c, args, att,
                 "value: the %d layers' block gather-attends captured back to back in a HIP "
                 "graph, replayed %d times (HIP events); steps: %d eager 4-layer plan steps after "
                 "%d warmup, per-layer HIP events" % (L, reps, n_steps, n_warm),
                 {"ms_per_step": round(ms_step, 4), "steps_per_s": round(1e3 / ms_step, 1),
                  "config": {"workload": "block61k: 128-token block selection, 4 layers "
                                         "[SPARSE, REUSE 0 x3]",
                             "batch": c.batch, "n_q_heads": c.n_q_heads,
                             "n_kv_heads": c.n_kv_heads, "head_dim": c.head_dim,
                             "ctx_len": c.ctx_len, "block_size": bs, "blocks_kept": c.k,
                             "modes": list(c.modes), "kv_dtype": c.dtype,
                             "parallelism": "single GPU"},
                  "kernels": kernels,
                  "layers_us": {"sparse": round(us_layer[0], 1),
                                "reuse": round(sum(us_layer[1:]) / (L - 1), 1),
                                "sparse_cold": round(cold["sparse_layer"], 1),
                                "dense": round(us_dense, 1)},
                  "plan_step_us": round(ms_step * 1e3, 1),
                  "all_dense_step_us": round(us_dense4, 1),
                  "plan_speedup_vs_all_dense": round(us_dense4 / (ms_step * 1e3), 2),
                  "omega_msr": 1.0,
                  "generation_s": round(gen_s, 1), "upload_s": round(up_s, 1),
                  "cpu_baseline": cpu})
    line["roofline"]["cold_frac_of_same_bytes_stream"] = round(cold["stream"] / cold["attend"], 4)
    print(json.dumps(line), flush=True)


def bench_indexer1m(args):
    """One sequence of 1048576 tokens, 32/8 heads, d 128, bf16, 8 layers:
    layers 0-1 DENSE, layers 2-7 SPARSE, each with its own lightning indexer
    (4 heads x 64 dims, keys projected from the layer's keys) and a top-2048
    shared by the 8 KV heads.  `value`: the gather-attend of the six sparse
    layers (8.39 MB each) captured back to back in a HIP graph; beside it
    the 8-layer mixed step against 8 dense layers, and Omega_MSR (the share
    of layers attending sparsely)."""
    import shutil
    import tempfile
    import sa_synth as S

    name = "indexer1m"
    c = S.CONFIGS[name]
    L = c.n_layers
    sparse_l = [l for l in range(L) if c.modes[l] == "sparse"]
    att_bytes = 2 * c.n_kv_heads * c.k * c.head_dim * 2 + c.k * 4 + c.n_q_heads * c.head_dim * 6
    w = S.Workload(name, args.seed)
    log("%s: generating %d layers (%.1f GB of KV)" % (name, L, L * c.kv_bytes() / 1e9))
    t0 = time.perf_counter()
    host = []
    for l in range(L):
        kh, vh, qh = w.k(l), w.v(l), w.q(l)
        ind = None
        if c.modes[l] == "sparse":
            ind = (w.indexer_q(l, qh), w.indexer_k(l, kh), w.indexer_w(l))
        host.append((kh, vh, qh, ind))
    gen_s = time.perf_counter() - t0
    cpu = None
    if args.cpu_seconds > 0:
        shm = tempfile.mkdtemp(prefix="sa_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm")
                               else None)
        try:
            for l in sparse_l:
                qi, ki, wi = host[l][3]
                np.savez(os.path.join(shm, "layer%d.npz" % l), qi=qi, ki=ki, wi=wi, q=host[l][2])
            cpu = config_cpu_baseline(name, args.seed, att_bytes * len(sparse_l), shm)
        finally:
            shutil.rmtree(shm, ignore_errors=True)

    import torch
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)

    def up(x):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return (t.view(torch.bfloat16) if t.dtype == torch.uint16 else t).to(dev)

    t0 = time.perf_counter()
    qs, ks, vs, qi, ki, wi = [], [], [], {}, {}, {}
    for l in range(L):
        kh, vh, qh, ind = host[l]
        ks.append(up(kh))
        vs.append(up(vh))
        qs.append(up(qh))
        if ind is not None:
            qi[l], ki[l], wi[l] = up(ind[0]), up(ind[1]), up(ind[2][None, :].copy())
        host[l] = None
    torch.cuda.synchronize()
    up_s = time.perf_counter() - t0
    del host
    outs = [torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32, device=dev)
            for _ in range(L)]
    largs = [T.layer_args(qs[l], ks[l], vs[l], T.SA_SCORE_INDEXER, c.k, q_idx=qi.get(l),
                          k_idx=ki.get(l), idx_w=wi.get(l), out=outs[l])[0]
             if l in qi else T.layer_args(qs[l], ks[l], vs[l], T.SA_SCORE_EXACT, c.k,
                                          out=outs[l])[0] for l in range(L)]
    idx = [torch.empty((c.batch, c.k), dtype=torch.int32, device=dev) for _ in range(L)]
    mixed = [T.SA_LAYER_DENSE if m == "dense" else T.SA_LAYER_SPARSE for m in c.modes]
    T.sa_plan_validate(mixed, list(c.src))
    ws = {m: T.WORKSPACES.get(dev, (name, m), max(T.sa_layer_workspace_size(largs[l], m)
                                                  for l in sparse_l))
          for m in (T.SA_LAYER_DENSE, T.SA_LAYER_SPARSE)}

    def layer(l, m):
        T.sa_decode_layer(largs[l], m, None if m == T.SA_LAYER_DENSE else idx[l], dev, ws[m])

    n_steps, n_warm = max(3, min(args.steps, 20)), max(1, min(args.warmup, 3))
    for _ in range(n_warm):
        for l in range(L):
            layer(l, mixed[l])
    torch.cuda.synchronize()
    for l in sparse_l:
        assert T.sa_check_indices(qs[l], ks[l], idx[l], T.SA_IDX_TOKEN_SHARED).tolist() == [0, 0]
    log("%s: timing %d 8-layer steps" % (name, n_steps))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(L + 1)] for _ in range(n_steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_steps):
        for l in range(L):
            ev[i][l].record()
            layer(l, mixed[l])
        ev[i][L].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / n_steps
    us_layer = [sum(e[l].elapsed_time(e[l + 1]) for e in ev) / n_steps * 1e3 for l in range(L)]
    us_dense8 = _ev_us(lambda: [layer(l, T.SA_LAYER_DENSE) for l in range(L)], 3, warm=1)
    reps = max(10, min(args.steps, 50))

    def attend(l):
        return lambda: T.sa_sparse_decode(qs[l], ks[l], vs[l], idx[l], out=outs[l],
                                          index_kind=T.SA_IDX_TOKEN_SHARED)

    us_att = _graph_us([attend(l) for l in sparse_l], reps)
    scores = [torch.empty((c.batch, c.ctx_len), dtype=torch.float32, device=dev) for _ in sparse_l]
    sel = torch.empty((c.batch, c.k), dtype=torch.int32, device=dev)
    n_sp = len(sparse_l)
    us_score = _ev_us(lambda: [T.sa_score(qs[l], ks[l], T.SA_SCORE_INDEXER, q_idx=qi[l],
                                          k_idx=ki[l], idx_w=wi[l], scores=scores[j])
                               for j, l in enumerate(sparse_l)], max(3, reps // n_sp)) / n_sp
    us_topk = _ev_us(lambda: [T.sa_topk(scores[j], c.k, idx_out=sel) for j in range(n_sp)],
                     max(3, reps // n_sp)) / n_sp
    torch.cuda.synchronize()
    score_bytes = c.ctx_len * c.indexer_dim * 2 + c.ctx_len * 4
    dense_bytes = 2 * c.n_kv_heads * c.ctx_len * c.head_dim * 2
    us_sparse = sum(us_layer[l] for l in sparse_l) / n_sp
    us_dense = sum(us_layer[l] for l in range(L) if l not in sparse_l) / (L - n_sp)
    att = _rate(att_bytes, us_att)
    kernels = {"sparse_attend": att, "indexer_score": _rate(score_bytes, us_score),
               "topk_1m": _rate(c.ctx_len * 4 + c.k * 4, us_topk),
               "dense_layer": _rate(dense_bytes, us_dense)}
    line = _line(name, c, args, att,
                 "value: the %d sparse layers' gather-attends captured back to back in a HIP "
                 "graph, replayed %d times (HIP events); steps: %d eager 8-layer steps after %d "
                 "warmup, per-layer HIP events" % (n_sp, reps, n_steps, n_warm),
                 {"ms_per_step": round(ms_step, 4), "steps_per_s": round(1e3 / ms_step, 2),
                  "config": {"workload": "indexer1m: one 1M-token sequence, 8 layers (2 dense, "
                                         "6 sparse with a 4x64 lightning indexer, top-2048 "
                                         "shared by the KV heads)",
                             "batch": c.batch, "n_q_heads": c.n_q_heads,
                             "n_kv_heads": c.n_kv_heads, "head_dim": c.head_dim,
                             "ctx_len": c.ctx_len, "k": c.k, "indexer_heads": c.indexer_heads,
                             "indexer_dim": c.indexer_dim, "modes": list(c.modes),
                             "kv_dtype": c.dtype, "parallelism": "single GPU"},
                  "kernels": kernels,
                  "layers_us": {"sparse": round(us_sparse, 1), "dense": round(us_dense, 1)},
                  "mixed_step_us": round(ms_step * 1e3, 1),
                  "all_dense_step_us": round(us_dense8, 1),
                  "mixed_speedup_vs_all_dense": round(us_dense8 / (ms_step * 1e3), 2),
                  "omega_msr": round(n_sp / L, 4),
                  "generation_s": round(gen_s, 1), "upload_s": round(up_s, 1),
                  "cpu_baseline": cpu})
    print(json.dumps(line), flush=True)


def hylra(args):
    """Layer-reuse policy on 8 layers of the llama32k shape.

    Queries and keys of layer l follow x_l = rho_l x_{l-1} + sqrt(1 - rho_l^2) z_l
    with the hylra32k schedule (a weakly correlated layer 4): the seeded
    hylra32k workload, generated on the host (untimed).
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
    w = S.Workload(c, args.seed)
    log("hylra: generating %d layers (%.1f GB of KV)" % (L, L * c.kv_bytes() / 1e9))
    qs, ks, vs = [], [], []
    for l in range(L):
        kd, vd, _, _ = upload_kv(w, l, dev)
        ks.append(kd)
        vs.append(vd)
        qs.append(torch.from_numpy(w.q(l)).view(torch.bfloat16).to(dev))
        log("hylra: layer %d generated" % l)
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
        "data": "synthetic: the seeded hylra32k workload (seed %d)" % args.seed,
        "provenance": provenance()}), flush=True)


def offload(args):
    """Index-guided offload on the block61k shape (batch 8, 32/8 heads, d 128,
    bf16, 61440 tokens = 480 blocks of 128, 24 blocks kept per row).

    Layer 0's cache is on the device; it selects blocks from min/max
    summaries.  Layers 1-3 keep their caches in pinned host memory and reuse
    layer 0's blocks: sa_gather_blocks fetches only those blocks, and dense
    decode over the gathered rows is their attention.  The seeded block61k
    workload (its four layers), generated on the host (untimed)."""
    import torch
    import sa_synth as S
    import top_sparse_decode_sa_amd as T

    T.lib()
    dev = torch.device("cuda", 0)
    c = S.CONFIGS["block61k"]
    B, Hq, Hkv, d, N, bs, nblk = (c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.ctx_len,
                                  c.block_size, c.k)
    w = S.Workload(c, args.seed)
    shape = (B, Hkv, N, d)
    log("offload: generating 4 layers (%.1f GB of KV, 3 layers in pinned host memory)" % (
        4 * c.kv_bytes() / 1e9))
    qs = [torch.from_numpy(w.q(l)).view(torch.bfloat16).to(dev) for l in range(4)]
    k0, v0, _, _ = upload_kv(w, 0, dev)
    host = []
    for l in range(1, 4):
        kh = torch.empty(shape, dtype=torch.bfloat16, pin_memory=True)
        vh = torch.empty(shape, dtype=torch.bfloat16, pin_memory=True)
        kh.copy_(torch.from_numpy(w.k(l)).view(torch.bfloat16))
        vh.copy_(torch.from_numpy(w.v(l)).view(torch.bfloat16))
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
        "data": "synthetic: the seeded block61k workload (seed %d)" % args.seed,
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
    if args.block61k:
        args.workload = "block61k"
    if args.indexer1m:
        args.workload = "indexer1m"
    seeded = {"block61k": bench_block61k, "batch128k": bench_batch128k,
              "indexer1m": bench_indexer1m}
    if args.gpus == 1 and args.workload in seeded:
        seeded[args.workload](args)
        return
    if args.gpus == 1 and args.nscale:
        nscale(args)
        return
    if args.gpus == 1 and args.perhead:
        bench_perhead(args)
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

    # the same step as the library's SPARSE layer call: the fused selection's
    # part kernel, then the merge of the parts' candidates and the
    # gather-attend in one launch (merge_attend_kernel)
    n_graph = N_QVAR * n_rep // math.gcd(N_QVAR, n_rep)
    largs = [T.layer_args(qd[v % N_QVAR], kds[v % n_rep], vds[v % n_rep], T.SA_SCORE_EXACT, c.k,
                          out=out)[0] for v in range(n_graph)]
    lws = torch.empty(max(1, T.sa_layer_workspace_size(largs[0], T.SA_LAYER_SPARSE)),
                      dtype=torch.uint8, device=dev)

    def layer_step(i):
        T.sa_decode_layer(largs[i % n_graph], T.SA_LAYER_SPARSE, idx, dev, lws)

    log("bench: warmup %d steps" % args.warmup)
    for i in range(args.warmup):
        step(i)
        layer_step(i)
    torch.cuda.synchronize()
    # the layer call selects and attends exactly as the two calls
    step(0)
    two_idx, two_out = idx.clone(), out.clone()
    layer_step(0)
    torch.cuda.synchronize()
    assert torch.equal(two_idx, idx) and torch.equal(two_out, out), "layer call differs from the two calls"

    # the timed steps: each step captured once per (query variant, cache
    # copy) as a HIP graph, replayed in turn; the layer call's graphs give
    # ms_per_step, the two calls' graphs the two-call figure beside it
    def timed(fn, name):
        graphs = []
        if not args.eager:
            for v in range(n_graph):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fn(v)
                graphs.append(g)
            for i in range(args.warmup):
                graphs[i % n_graph].replay()
            torch.cuda.synchronize()
            # a replayed step selects and attends exactly as the eager one
            graphs[0].replay()
            g_idx, g_out = idx.clone(), out.clone()
            fn(0)
            torch.cuda.synchronize()
            assert torch.equal(g_idx, idx) and torch.equal(g_out, out), \
                "graph replay of the %s differs from eager" % name
        log("bench: timing %d steps of the %s (%s)" % (args.steps, name,
                                                      "eager" if args.eager else "graph replay"))
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(args.steps):
            if args.eager:
                fn(i)
            else:
                graphs[i % n_graph].replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t_start) * 1e3 / args.steps

    ms_step = timed(layer_step, "SPARSE layer call")
    ms_step_two = timed(step, "two calls")

    # The gather-attend alone (the headline): every (query variant, cache
    # copy) pair's own index set, selected once, then the n_graph attends
    # captured back to back in one graph whose replays are timed with events
    # on the launch stream.  Consecutive attends read different copies
    # (n_graph x 43.65 MB > the 256 MB last-level cache), so each finds its
    # rows evicted, as in the step.
    idx_v = [torch.empty_like(idx) for _ in range(n_graph)]
    out_v = [torch.empty_like(out) for _ in range(n_graph)]
    for v in range(n_graph):
        T.sa_select(qd[v % N_QVAR], kds[v % n_rep], c.k, idx_out=idx_v[v])

    def attends():
        for v in range(n_graph):
            T.sa_sparse_decode(qd[v % N_QVAR], kds[v % n_rep], vds[v % n_rep], idx_v[v], out=out_v[v])

    attends()
    torch.cuda.synchronize()
    eager_out = [o.clone() for o in out_v]
    g_att = None
    if not args.eager:
        g_att = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_att):
            attends()
        g_att.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a_, b_) for a_, b_ in zip(out_v, eager_out)), \
            "attend graph replay differs from eager"
    n_att_rep = max(25, args.steps // n_graph)
    for _ in range(3):
        g_att.replay() if g_att else attends()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_att_rep):
        g_att.replay() if g_att else attends()
    e1.record()
    torch.cuda.synchronize()
    ms_attend = e0.elapsed_time(e1) / (n_att_rep * n_graph)

    # the same launches' reads without their arithmetic (sa_gather_read: the
    # same plan, index loads and row loads), timed the same way: the floor
    # for this gather-attend on these rows
    gsink = torch.zeros(1, dtype=torch.int32, device=dev)

    def gathers():
        for v in range(n_graph):
            T.sa_gather_read(qd[v % N_QVAR], kds[v % n_rep], vds[v % n_rep], idx_v[v], gsink)

    gathers()
    torch.cuda.synchronize()
    g_gat = None
    if not args.eager:
        g_gat = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_gat):
            gathers()
    for _ in range(3):
        g_gat.replay() if g_gat else gathers()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n_att_rep):
        g_gat.replay() if g_gat else gathers()
    e1.record()
    torch.cuda.synchronize()
    ms_gather = e0.elapsed_time(e1) / (n_att_rep * n_graph)

    # per-call durations inside eager steps: HIP events on the launch stream
    # between the two calls (each event pair also holds its launch's
    # dispatch, a few us)
    n_ev = min(args.steps, 100)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    torch.cuda.synchronize()
    t_ev = time.perf_counter()
    for i in range(n_ev):
        step(i, events[i])
    torch.cuda.synchronize()
    ms_step_eager = (time.perf_counter() - t_ev) * 1e3 / n_ev
    ms_select = sum(e[0].elapsed_time(e[1]) for e in events) / n_ev
    ms_attend_in_step = sum(e[1].elapsed_time(e[2]) for e in events) / n_ev

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

    # the device's streaming read rate (sa_stream_read over 8 GiB)
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

    nbytes = step_bytes(c)
    att_bytes = nbytes["sparse_attend"]

    # cache-cold single launches: before each, a 1 GiB read evicts L2 and the
    # 256 MB last-level cache; the gather-attend, and beside it the same
    # number of bytes read by the library's streaming read (the floor a
    # single launch of this size can reach on this device)
    cold = None
    if args.cold_iters > 0:
        flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        sbuf = torch.empty(att_bytes // 16 * 16, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        cout = torch.empty_like(out)
        times = {"sparse": [], "stream": []}
        for i in range(args.cold_iters + 2):
            for name in ("sparse", "stream"):
                flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                if name == "sparse":
                    T.sa_sparse_decode(qd[0], kd, vd, idx_v[0], out=cout)
                else:
                    T.sa_stream_read(sbuf, sink)
                e1.record()
                torch.cuda.synchronize()
                if i >= 2:
                    times[name].append(e0.elapsed_time(e1))
        del flush, sbuf
        cold = {name: float(np.median(v)) for name, v in times.items()}

    step_total = nbytes["select"] + att_bytes

    def kern(name, ms, nb=None):
        if ms is None:
            return None
        nb = nbytes[name] if nb is None else nb
        g = nb / (ms * 1e-3) / 1e9
        return {"bytes": nb, "us": round(ms * 1e3, 3), "gbps": round(g, 1),
                "frac": round(g / HBM_PEAK_GBPS, 4)}

    att = kern("sparse_attend", ms_attend)
    kernels = {"sparse_attend": att,
               "gather_read_same_rows": kern("sparse_attend", ms_gather),
               "sparse_attend_in_step": kern("sparse_attend", ms_attend_in_step),
               "select": kern("select", ms_select),
               "score_exact": kern("score_exact", ms_score), "topk": kern("topk", ms_topk),
               "dense_decode": kern("dense_decode", ms_dense)}
    floor = None
    if cold:
        kernels["sparse_attend_cold"] = kern("sparse_attend", cold["sparse"])
        floor = kern("sparse_attend", cold["stream"], nb=att_bytes // 16 * 16)
        kernels["stream_read_same_bytes_cold"] = floor
    roof = {"bound": "hbm", "achieved": att["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": att["frac"], "traffic": read_traffic("sparse_attend"),
            "kernel": "sparse_attend", "bytes_per_launch": att_bytes}
    if stream:
        roof["frac_of_stream_read"] = round(att["gbps"] / stream["gbps"], 4)
    # the gather-attend against its own reads alone (sa_gather_read)
    roof["frac_of_gather_read"] = round(ms_gather / ms_attend, 4)
    if cold:
        # the cold single launch against a cold streaming read of its bytes
        roof["cold_frac_of_same_bytes_stream"] = round(cold["stream"] / cold["sparse"], 4)

    cpu = None
    if args.cpu_seconds > 0:
        log("bench: oracle cpu baseline (bounded to %.0f s)" % args.cpu_seconds)
        idx_host = idx_v[0].cpu().numpy()
        att_s, step_s, done, total = cpu_baseline(w, q_host, k_host, v_host, idx_host,
                                                  args.cpu_seconds)
        cpu = {"value": round(att_bytes / att_s / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "steps_per_s": round(1.0 / att_s, 4),
               "full_step_steps_per_s": round(1.0 / step_s, 4),
               "sample": "fp64 numpy oracle, one thread: selected-set attention over the GPU's "
                         "index sets of %d of the %d (sequence, KV head) rows of one step, scaled "
                         "by %d/%d; full_step adds the oracle's exact scores and top-k" % (
                             done, total, total, done)}
        cpu.update(host_cpu())

    line = {
        "metric": "sparse-decode attn: achieved HBM GB/s (% of peak) + decode steps/s at 50x",
        "value": att["gbps"],
        "unit": "GB/s",
        "hbm_frac": att["frac"],
        "attend_us": att["us"],
        "attend_steps_per_s": round(1e3 / ms_attend, 1),
        "steps_per_s": round(1e3 / ms_step, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "timing": ("value: the gather-attend alone, %d attends over %d cache copies captured back "
                   "to back in a HIP graph, replayed %d times between HIP events; ms_per_step and "
                   "steps_per_s: the K timed decode steps (the SPARSE layer call: exact selection "
                   "+ gather-attend), each a replayed HIP graph" % (n_graph, n_rep, n_att_rep)),
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
        "step": {"what": "sa_decode_layer(SPARSE): the fused exact selection's part kernel "
                         "(scores kept on chip, each part's top-k), then the merge of the parts' "
                         "candidates and the gather-attend in one launch",
                 "ms_per_step": round(ms_step, 4), "steps_per_s": round(1e3 / ms_step, 1),
                 "gbps": round(step_total / (ms_step * 1e-3) / 1e9, 1),
                 "frac": round(step_total / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                 "bytes": step_total,
                 "timing": "eager launches" if args.eager else "each step a replayed HIP graph",
                 "two_calls": {"what": "sa_select -> sa_sparse_decode (the same index list and "
                                       "output)", "ms_per_step": round(ms_step_two, 4),
                               "steps_per_s": round(1e3 / ms_step_two, 1),
                               "ms_per_step_eager_with_events": round(ms_step_eager, 4)}},
        "kernels": kernels,
        "sparse_over_dense_speedup": (round(ms_dense / ms_attend, 2) if ms_dense else None),
        "stream_read": stream,
        "cpu_baseline": cpu,
        "provenance": provenance(clocks=not args.profile),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
