"""Benchmark: ProxyAttn block-sparse causal prefill on one MI355X.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload llama8b_128k_g4]

One step = one pass of the whole method over one layer of synthetic input
already resident in HBM: proxy_pool -> proxy_score -> budget -> block_select
-> sparse attention (pxa_prefill).  Prints one JSON line with the step latency
(ms), the dense-attention baseline of the same kernel family, the speedup,
the estimation share, the kept-block density, per-stage times, the roofline
of the dominant kernel (sparse attention, MFMA-bound) and the CPU oracle timed
on a bounded sample of the same workload (a reported baseline only).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill-attn ms & speedup vs dense @128K; MFMA util on kept blocks"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
B = 128


def parse():
    from synth.configs import CONFIGS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1, help="GPUs (only 1 is supported)")
    ap.add_argument("--steps", type=int, default=10, help="timed steps (whole method per step)")
    ap.add_argument("--warmup", type=int, default=3, help="untimed steps before the timed ones")
    ap.add_argument("--workload", default="llama8b_128k_g4", choices=sorted(CONFIGS),
                    help="layer shape, length, proxies and gamma of the synthetic input")
    ap.add_argument("--gamma", type=float, default=None, help="override the workload's gamma")
    ap.add_argument("--dense-reps", type=int, default=3,
                    help="timed runs of the dense kernel (the speedup denominator)")
    ap.add_argument("--score-stride", type=int, default=1,
                    help="sequence-level skip of the proxy scoring: score every s-th query "
                         "(1, 2 or 4; 1 = every query, the default)")
    ap.add_argument("--skip-threshold", type=float, default=0.0,
                    help="BLASST running-max skip inside the attention (0 = off, the default)")
    ap.add_argument("--budget", default="dynamic:1",
                    help="budget variant: dynamic:M (probe the last M query blocks; the method's "
                         "own budget, M=1 by default), fixed:K or ratio:R")
    ap.add_argument("--seq-len", type=int, default=None,
                    help="override the workload's N (any length >= 1; when 128 does not divide "
                         "it the last block is partial)")
    ap.add_argument("--batch-lens", default=None,
                    help="comma-separated sequence lengths: time one pxa_prefill_batch call over "
                         "them (heads, dims, proxies and gamma of --workload) against one "
                         "pxa_prefill_ex call per sequence, and print that line instead")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the timed sample of the CPU oracle")
    ap.add_argument("--no-sdpa", action="store_true",
                    help="skip the context timing of torch's flash SDPA at the same shape")
    ap.add_argument("--cpu-budget-s", type=float, default=30.0,
                    help="approximate CPU seconds for the oracle sample")
    ap.add_argument("--no-live-traffic", action="store_true",
                    help="skip the two rocprofv3 counter passes that measure the sparse kernel's "
                         "HBM traffic in this run (the committed profile is used instead)")
    ap.add_argument("--profile", action="store_true",
                    help="short pass for hardware counters: one 256 MiB device copy (counter "
                         "calibration), one warm pxa_prefill, then --steps passes of the stages")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["block_sparse_long_proxy_amd/csrc/fa_prefill.hip",
                  "block_sparse_long_proxy_amd/csrc/pxa_device.hpp"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(workload, config):
    """HBM bytes per sparse-attention launch from the committed rocprofv3
    counter summary of this workload, or None if it is missing, was taken on
    another configuration (inputs, gamma, budget, stride, skip) or on
    different kernel sources."""
    try:
        with open(os.path.join(PROFILE_DIR, f"fa_prefill_sparse_{workload}.md")) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    kv = {}
    for line in lines:
        if ":" in line:
            k, v = line.split(":", 1)
            kv.setdefault(k.strip(), v.strip())
    if kv.get("workload") != workload or kv.get("source_sha256") != kernel_source_hash():
        return None
    if kv.get("config") != json.dumps(config, sort_keys=True):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _is_sparse_attention(kernel_name):
    """fa_prefill_kernel<D, DENSE, SKIP> with DENSE false."""
    tag = "fa_prefill_kernel<"
    if tag not in kernel_name:
        return False
    args = kernel_name.split(tag, 1)[1].split(">", 1)[0].split(",")
    return len(args) == 3 and args[1].strip() == "false"


def live_traffic(a, timeout_s=180):
    """HBM bytes per launch of the sparse attention kernel, measured in this run.

    Two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE) run a child
    `bench.py --profile` of the same configuration. Each counter is averaged
    over the kernel's launches and scaled by what it reads for the 256 MiB
    device copy the child makes first (KiB per launch). Returns None if
    rocprofv3 is missing or a pass fails or times out.
    """
    import csv
    import glob
    import shutil
    import signal
    import subprocess
    import tempfile
    prof = shutil.which("rocprofv3")
    if prof is None:
        return None
    child = [sys.executable, os.path.abspath(__file__), "--workload", a.workload, "--profile",
             "--steps", "1", "--budget", a.budget, "--score-stride", str(a.score_stride),
             "--skip-threshold", repr(a.skip_threshold)]
    if a.gamma is not None:
        child += ["--gamma", repr(a.gamma)]
    if a.seq_len is not None:
        child += ["--seq-len", str(a.seq_len)]
    env = dict(os.environ, TMPDIR="/tmp")
    total = 0.0
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        log(f"counter pass {counter} (rocprofv3, child bench.py --profile)")
        with tempfile.TemporaryDirectory(dir="/tmp") as d:
            cmd = [prof, "--pmc", counter, "--output-format", "csv", "-d", d, "-o", "p", "--"] + child
            # the child's log lines go to this process's stderr; stdout stays the JSON line's
            p = subprocess.Popen(cmd, cwd="/tmp", env=env, stdout=subprocess.DEVNULL,
                                 start_new_session=True)
            try:
                p.wait(timeout=timeout_s)
            except subprocess.TimeoutExpired:
                os.killpg(p.pid, signal.SIGKILL)
                p.wait()
                log(f"counter pass {counter} timed out")
                return None
            # the profiler itself may end with an error after a complete run; the
            # results file decides
            files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
            if not files:
                log(f"counter pass {counter}: no results (rc {p.returncode})")
                return None
            copy_kib, kernel_kib = None, []
            with open(files[0]) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] != counter:
                        continue
                    if "copyBuffer" in r["Kernel_Name"] and copy_kib is None:
                        copy_kib = float(r["Counter_Value"])
                    elif _is_sparse_attention(r["Kernel_Name"]):
                        kernel_kib.append(float(r["Counter_Value"]))
            if not copy_kib or not kernel_kib:
                log(f"counter pass {counter}: calibration or kernel rows missing")
                return None
            total += sum(kernel_kib) / len(kernel_kib) * 1024.0 * (262144.0 / copy_kib)
    return total


def cpu_baseline(cfg, x, samples, n_kept, gpu_csr, budget_s=20.0, last_blocks=1,
                 budget_kind="dynamic", score_stride=1, gamma=None, budget_param=None):
    """Time the CPU oracle (float64 NumPy, as it stands) and scale it to the full step.

    Pooling and, for the dynamic budget, the masses of every head are timed in
    full (heads spread over a thread pool); the proxy scores of a sample of
    rows of every proxy (scaled by causal tiles), the selection of those rows
    (scaled by rows) and the sparse attention of a few (head, row) pairs on the
    GPU's own mask (scaled by kept tiles) are sampled.  The same oracle
    intermediates then check the GPU's mask on the sampled rows against the
    oracle's own chain (its proxies, scores, ranking and budgets).
    `samples`: list of (h, I, kept block indices); gpu_csr: (row_ptr, col_idx, k_h);
    budget_param: the blocks of a fixed budget or the ratio of a ratio budget.
    """
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import proxyattn as O
    from synth import bf16_bits_to_f32

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(cores)
    except Exception:  # pragma: no cover
        pass
    H, Hkv, N, d, G, nb = (cfg.num_heads, cfg.num_kv_heads, cfg.seq_len, cfg.head_dim,
                           cfg.num_proxies, cfg.nb)
    f64 = lambda a: bf16_bits_to_f32(a).astype(np.float64)  # noqa: E731
    scale = cfg.scale
    est = {}
    t_all = time.perf_counter()
    row_k = ((lambda h, I: budget_param) if budget_kind == "fixed" else
             (lambda h, I: O.ratio_count(I, budget_param)))

    # pooling, every token of every proxy
    t = time.perf_counter()
    qbar = np.zeros((G, N, d))
    kbar = np.zeros((G, N, d))
    for g in range(G):
        heads, kvs = O.group_query_heads(g, H, G), O.group_kv_heads(g, H, Hkv, G)
        qg, kg = O.proxy_pool(f64(x["q"][heads]), f64(x["k"][kvs]), 1)
        qbar[g], kbar[g] = qg[0], kg[0]
    est["pool"] = time.perf_counter() - t

    # proxy scores: the last row and a spread of rows of every proxy
    rows = sorted({nb - 1} | {(c * nb) // 8 for c in range(1, 8)})
    S_ref = np.full((G, nb, nb), -np.inf)
    t = time.perf_counter()
    for g in range(G):
        for I in rows:
            S_ref[g, I, : I + 1] = O.proxy_score_row(qbar[g], kbar[g], I, B, scale, score_stride)
    tiles = G * sum(I + 1 for I in rows)
    est["score"] = (time.perf_counter() - t) * (G * nb * (nb + 1) / 2) / tiles
    del qbar, kbar

    # budgets: the masses of every head (threads over heads), then the cumulative
    # mass along the group's ranking of the last row
    k_ref = None
    if budget_kind == "dynamic":
        def masses_of(h):
            q_h, k_h = f64(x["q"][h]), f64(x["k"][O.kv_head_of(h, H, Hkv)])
            if last_blocks == 1:
                return O.last_block_masses(q_h, k_h, B, scale)
            return O.last_blocks_masses(q_h, k_h, B, scale, last_blocks)
        t = time.perf_counter()
        with ThreadPoolExecutor(cores) as ex:
            masses = list(ex.map(masses_of, range(H)))
        orders = [O.rank_blocks(S_ref[g, nb - 1], nb - 1) for g in range(G)]
        k_ref = [O.budget_from_masses(masses[h], orders[O.group_of(h, H, G)], gamma)
                 for h in range(H)]
        est["budget"] = time.perf_counter() - t
    else:
        est["budget"] = 0.0

    # selection of the sampled rows of every head (scaled by rows)
    t = time.perf_counter()
    sel = {}
    for h in range(H):
        for I in rows:
            kk = row_k(h, I) if k_ref is None else k_ref[h]
            sel[h, I] = O.select_row(S_ref[O.group_of(h, H, G), I], I, kk)
    est["select"] = (time.perf_counter() - t) * nb / len(rows)

    done, spent = 0, 0.0
    heads = {}
    for h, I, cols in samples:
        kv = h // (H // Hkv)
        if h not in heads:
            heads = {h: (f64(x["q"][h]), f64(x["k"][kv]), f64(x["v"][kv]))}
        qh, kk, vv = heads[h]
        t = time.perf_counter()
        O.sparse_attention_row(qh, kk, vv, cols, I, B, scale)
        spent += time.perf_counter() - t
        done += len(cols)
        if spent > budget_s * 0.5:
            break
    est["sparse"] = spent * n_kept / max(done, 1)

    # the GPU's mask on the sampled rows against the oracle's chain: a block may
    # differ only within 1e-3 relative of the oracle's score across the cut
    rp, ci, kh_gpu = gpu_csr
    kh_gpu = [None] * H if kh_gpu is None else kh_gpu
    differ = gap_ok = 0
    worst = 0.0
    total = 0
    for (h, I), want in sel.items():
        got = set(ci[rp[h * nb + I]:rp[h * nb + I + 1]].tolist())
        want = set(want.tolist())
        total += I + 1
        s_row = S_ref[O.group_of(h, H, G), I]
        order = O.rank_blocks(s_row, I)
        kk = min(int(row_k(h, I) if k_ref is None else k_ref[h]), I + 1)
        for J in want ^ got:
            differ += 1
            c = kk if J in want else kk - 1
            if 0 <= c <= I and order[c] != J:
                gap = abs(s_row[J] - s_row[order[c]]) / max(abs(s_row[J]), abs(s_row[order[c]]))
                if gap < 1e-3:
                    gap_ok += 1
                    worst = max(worst, gap)
    mask = {"rows": rows, "heads": H, "causal_blocks": total,
            "agreement": round(1.0 - differ / max(total, 1), 7), "blocks_differing": differ,
            "within_gap_rule": gap_ok, "outside_gap_rule": differ - gap_ok,
            "worst_gap_within_rule": float(worst),
            "budgets_equal_to_oracle": None if k_ref is None else
            int(np.sum(np.asarray(k_ref) == np.asarray(kh_gpu)))}
    return {
        "value": sum(est.values()) * 1e3, "unit": "ms", "cores": int(cores), "kind": "oracle",
        "sample": (f"float64 NumPy oracle on {cores} threads, reported baseline only: pooling of "
                   f"every token and the masses of all {H} heads timed in full; proxy scores of "
                   f"rows {rows} of every proxy, their selection, and sparse attention of {done} "
                   f"kept tiles of the GPU mask timed on that sample and scaled to the full step "
                   f"by causal tiles, rows and kept tiles"),
        "stage_s": {k: round(v, 3) for k, v in est.items()},
        "wall_s": round(time.perf_counter() - t_all, 2),
        "cpu_model": _cpu_model(),
    }, mask


def _cpu_model():
    """Model name of the host CPU (first entry of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_batch(a, wl):
    """Several sequences of the workload's layer shape in one pxa_prefill_batch
    call (stored one after another, fused workspace), timed against one
    pxa_prefill_ex call per sequence on the same buffers and against the batch
    call in a workspace for one sequence (sequences in turn)."""
    import dataclasses
    import numpy as np
    import torch
    import block_sparse_long_proxy_amd as pxa
    from synth import generate

    lens = [int(t) for t in a.batch_lens.split(",") if t]
    gamma = a.gamma if a.gamma is not None else wl.gamma
    H, Hkv, d, G = wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.num_proxies
    cfg = pxa.Config(H, Hkv, max(lens), d, G, gamma)
    opts = dataclasses.replace(pxa.Options.dynamic(), score_stride=a.score_stride,
                               skip_threshold=a.skip_threshold)
    log(f"generating {len(lens)} sequences of {wl.name}'s shape: {lens}")
    xs = [generate(wl.with_(name=f"{wl.name}_seq{i}", seq_len=n, seed=wl.seed + 1000 + i,
                            n_needles=min(n, wl.n_needles))) for i, n in enumerate(lens)]
    flat = {n: torch.cat([torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).reshape(-1)
                          for x in xs]).cuda() for n in ("q", "k", "v")}
    del xs
    o = torch.empty_like(flat["q"])
    ws = torch.empty(pxa.pxa_batch_workspace_bytes(cfg, opts, lens), dtype=torch.uint8,
                     device="cuda")
    single_bytes = pxa.pxa_workspace_bytes_ex(cfg, opts)
    stream = torch.cuda.current_stream()

    def batched():        # fused: one set of launches per group of sequences
        pxa.pxa_prefill_batch(cfg, opts, lens, flat["q"], flat["k"], flat["v"], o, ws)

    def batched_seq():    # a workspace for one sequence: the call runs them in turn
        pxa.pxa_prefill_batch(cfg, opts, lens, flat["q"], flat["k"], flat["v"], o, ws,
                              ws_bytes=single_bytes)

    views = []
    qo = ko = 0
    for n in lens:
        c = pxa.Config(H, Hkv, n, d, G, gamma)
        views.append((c, flat["q"][qo:qo + H * n * d], flat["k"][ko:ko + Hkv * n * d],
                      flat["v"][ko:ko + Hkv * n * d], o[qo:qo + H * n * d]))
        qo += H * n * d
        ko += Hkv * n * d

    def one_by_one():
        for c, q, k, v, oo in views:
            pxa.pxa_prefill_ex(c, opts, q, k, v, oo, ws)

    def timed(fn):
        for _ in range(a.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(a.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps

    ms_batch = timed(batched)
    ob = o.clone()
    ms_single = timed(one_by_one)
    same = bool(torch.equal(ob, o))
    ms_seq = timed(batched_seq) if single_bytes < ws.numel() else None
    # the fused call captured once in a HIP graph and replayed (launch costs gone)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        batched()
    ms_graph = timed(graph.replay)
    graph_same = bool(torch.equal(ob, o))
    log(f"fused batch {ms_batch:.3f} ms, one call per sequence {ms_single:.3f} ms, "
        f"batch in a one-sequence workspace {ms_seq}, identical {same}")
    tokens = sum(lens)
    print(json.dumps({
        "metric": "batched ProxyAttn prefill (pxa_prefill_batch) ms per call",
        "value": round(ms_batch, 3), "unit": "ms", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_batch, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generator, bf16, inputs resident in HBM)",
        "config": {"workload": f"{len(lens)} sequences of the {wl.name} layer shape",
                   "num_heads": H, "num_kv_heads": Hkv, "head_dim": d, "num_proxies": G,
                   "gamma": gamma, "seq_lens": lens, "score_stride": a.score_stride},
        "tokens": tokens, "tokens_per_s": round(tokens / (ms_batch * 1e-3), 1),
        "one_call_per_sequence_ms": round(ms_single, 3),
        "batch_in_one_sequence_workspace_ms": None if ms_seq is None else round(ms_seq, 3),
        "fused_graph_replay_ms": round(ms_graph, 3),
        "graph_replay_identical": graph_same,
        "speedup_vs_one_call_per_sequence": round(ms_single / ms_batch, 3),
        "workspace_bytes": {"fused": int(ws.numel()), "one_sequence": int(single_bytes)},
        "outputs_identical_to_one_call_per_sequence": same,
    }), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "only --gpus 1 is supported: the library runs the method on "
                          "one GPU and has no multi-GPU path",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    import numpy as np
    import torch
    import block_sparse_long_proxy_amd as pxa
    from synth import get_config, generate, input_digest

    wl = get_config(a.workload)
    if a.batch_lens:
        return bench_batch(a, wl)
    if a.seq_len is not None:
        wl = wl.with_(seq_len=a.seq_len, n_needles=min(a.seq_len, wl.n_needles),
                      description=f"{wl.description} with N={a.seq_len}")
    gamma = a.gamma if a.gamma is not None else wl.gamma
    cfg = pxa.Config(wl.num_heads, wl.num_kv_heads, wl.seq_len, wl.head_dim, wl.num_proxies, gamma)
    H, Hkv, N, d, G, nb = cfg.num_heads, cfg.num_kv_heads, cfg.seq_len, cfg.head_dim, cfg.num_proxies, cfg.nb
    log(f"generating {wl.name}: H={H} Hkv={Hkv} N={N} d={d} G={G} gamma={gamma}")
    t0 = time.time()
    x = generate(wl)
    digest = input_digest(x["q"], x["k"], x["v"])[:16]
    log(f"generated in {time.time() - t0:.1f}s digest {digest}")
    dev = {n: torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v")}
    torch.cuda.synchronize()
    kind, _, val = a.budget.partition(":")
    budget = {"dynamic": lambda: pxa.Options.dynamic(int(val or 1)),
              "fixed": lambda: pxa.Options.fixed(int(val)),
              "ratio": lambda: pxa.Options.ratio_of(float(val))}[kind]()
    import dataclasses
    budget = dataclasses.replace(budget, score_stride=a.score_stride,
                                 skip_threshold=a.skip_threshold)
    budget_desc = {"mode": kind, **({"last_blocks": budget.last_blocks} if kind == "dynamic" else
                                    {"blocks": budget.fixed_blocks} if kind == "fixed" else
                                    {"ratio": budget.ratio})}
    attn = pxa.ProxyAttn(cfg, budget)
    o = torch.empty_like(dev["q"])
    stream = torch.cuda.current_stream()
    L = attn.layout
    bws_bytes = pxa.pxa_budget_workspace_bytes_ex(cfg, budget)

    def budget_stage():
        if kind != "ratio":
            pxa.pxa_budget_estimate_ex(cfg, budget, dev["q"], dev["k"], attn.scores, attn.k_h,
                                       attn.masses, attn.ws[L.budget_ws:], ws_bytes=bws_bytes)

    def select_stage():
        pxa.pxa_block_select_ex(cfg, budget, attn.scores, None if kind == "ratio" else attn.k_h,
                                attn.row_ptr, attn.col_idx, attn.ws[L.select_ws:],
                                ws_bytes=pxa.pxa_select_workspace_bytes(cfg),
                                row_order=attn.row_order)

    if a.profile:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)      # calibration: 256 MiB read + 256 MiB written
        attn(dev["q"], dev["k"], dev["v"], out=o)
        for _ in range(a.steps):
            pxa.pxa_proxy_pool(cfg, dev["q"], dev["k"], attn.qbar, attn.kbar, attn.qexp, attn.kexp)
            pxa.pxa_proxy_score_ex(cfg, budget, attn.qbar, attn.kbar, attn.qexp, attn.kexp,
                                   attn.scores)
            budget_stage()
            select_stage()
            pxa.pxa_sparse_prefill_ex(cfg, budget, dev["q"], dev["k"], dev["v"], attn.row_ptr, attn.col_idx, o,
                                   row_order=attn.row_order)
        torch.cuda.synchronize()
        log(f"profile pass done: kept blocks {int(attn.row_ptr[-1])}")
        return

    # whole-step timing
    for _ in range(a.warmup):
        attn(dev["q"], dev["k"], dev["v"], out=o)
    torch.cuda.synchronize()
    log("warmup done")
    t_start = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(a.steps):
        attn(dev["q"], dev["k"], dev["v"], out=o)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / a.steps
    ms_step = ev0.elapsed_time(ev1) / a.steps
    log(f"pxa_prefill: {ms_step:.3f} ms/step (host wall {wall_ms:.3f})")

    # per-stage timing with the same kernels, events on the launch stream
    names = ["pool", "score", "budget", "select", "sparse"]
    acc = {n: 0.0 for n in names}
    reps = max(1, a.steps)
    for r in range(reps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        evs[0].record(stream)
        pxa.pxa_proxy_pool(cfg, dev["q"], dev["k"], attn.qbar, attn.kbar, attn.qexp, attn.kexp)
        evs[1].record(stream)
        pxa.pxa_proxy_score_ex(cfg, budget, attn.qbar, attn.kbar, attn.qexp, attn.kexp,
                               attn.scores)
        evs[2].record(stream)
        budget_stage()
        evs[3].record(stream)
        select_stage()
        evs[4].record(stream)
        pxa.pxa_sparse_prefill_ex(cfg, budget, dev["q"], dev["k"], dev["v"], attn.row_ptr, attn.col_idx, o,
                               row_order=attn.row_order)
        evs[5].record(stream)
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            acc[n] += evs[i].elapsed_time(evs[i + 1])
    stage = {n: acc[n] / reps for n in names}
    log("stages ms: " + " ".join(f"{n}={v:.3f}" for n, v in stage.items()))

    # dense baseline, same kernel family
    od = torch.empty_like(dev["q"])
    pxa.pxa_dense_prefill(cfg, dev["q"], dev["k"], dev["v"], od)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.dense_reps):
        pxa.pxa_dense_prefill(cfg, dev["q"], dev["k"], dev["v"], od)
    e1.record(stream)
    torch.cuda.synchronize()
    dense_ms = e0.elapsed_time(e1) / a.dense_reps
    log(f"dense: {dense_ms:.3f} ms")

    # the running-max skip is an approximation: its output against the same
    # mask without the skip, and the dense kernel with the skip alone (context)
    skip_cmp = None
    if a.skip_threshold > 0:
        o_ref = torch.empty_like(o)
        pxa.pxa_sparse_prefill(cfg, dev["q"], dev["k"], dev["v"], attn.row_ptr, attn.col_idx,
                               o_ref, row_order=attn.row_order)
        pxa.pxa_sparse_prefill_ex(cfg, budget, dev["q"], dev["k"], dev["v"], attn.row_ptr,
                                  attn.col_idx, o, row_order=attn.row_order)
        torch.cuda.synchronize()
        diff = (o.float() - o_ref.float()).abs()
        e0.record(stream)
        for _ in range(a.dense_reps):
            pxa.pxa_dense_prefill_ex(cfg, budget, dev["q"], dev["k"], dev["v"], od)
        e1.record(stream)
        torch.cuda.synchronize()
        skip_cmp = {"threshold": a.skip_threshold,
                    "output_vs_no_skip_max_abs": round(float(diff.max()), 5),
                    "output_vs_no_skip_mean_abs": round(float(diff.mean()), 7),
                    "dense_with_skip_ms": round(e0.elapsed_time(e1) / a.dense_reps, 3)}
        del o_ref, diff
        log(f"running-max skip: {skip_cmp}")

    # context only: torch's own fused causal attention (flash backend) at the same shape,
    # to show the dense denominator is not a weak baseline
    sdpa = None
    if not a.no_sdpa and wl.dtype == "bf16":
        try:
            from torch.nn.attention import sdpa_kernel, SDPBackend
            import torch.nn.functional as F
            qq, kk, vv = dev["q"][None], dev["k"][None], dev["v"][None]
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                F.scaled_dot_product_attention(qq, kk, vv, is_causal=True, enable_gqa=True)
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(a.dense_reps):
                    F.scaled_dot_product_attention(qq, kk, vv, is_causal=True, enable_gqa=True)
                e1.record(stream)
            torch.cuda.synchronize()
            sdpa = {"ms": round(e0.elapsed_time(e1) / a.dense_reps, 3),
                    "what": "torch.nn.functional.scaled_dot_product_attention, flash backend, "
                            "is_causal, enable_gqa, same bf16 inputs"}
            log(f"torch flash SDPA: {sdpa['ms']:.3f} ms")
        except Exception as e:  # a build without the flash backend: report, do not fail
            sdpa = {"ms": None, "error": repr(e)[:200]}

    # mask statistics
    rp = attn.row_ptr.cpu().numpy().astype(np.int64)
    kh = attn.k_h.cpu().numpy()
    n_kept = int(rp[-1])
    n_diag = H * nb
    causal_half_blocks = H * nb * nb / 2.0
    density = (n_kept - 0.5 * n_diag) / causal_half_blocks
    f_kept = (n_kept - n_diag) * 4.0 * B * B * d + n_diag * 2.0 * B * B * d
    f_dense = 2.0 * N * N * d * H
    f_score = G * (nb * (nb + 1) / 2) * 2.0 * B * B * d / a.score_stride
    tflops = lambda f, ms: f / (ms * 1e-3) / 1e12  # noqa: E731
    kept_tflops = tflops(f_kept, stage["sparse"])
    # Estimation cost inside the whole-method call: the step minus its sparse
    # attention kernel (pxa_prefill runs the budget probe inside the score
    # launch, so the standalone stage times above add up to more than it pays).
    est_ms = ms_step - stage["sparse"]
    est_stages_ms = stage["pool"] + stage["score"] + stage["budget"] + stage["select"]

    # the skip is an approximation: compare its mask with the every-query mask
    stride_cmp = None
    if a.score_stride > 1:
        full = dataclasses.replace(budget, score_stride=1)
        S1 = torch.empty_like(attn.scores)
        pxa.pxa_proxy_score_ex(cfg, full, attn.qbar, attn.kbar, attn.qexp, attn.kexp, S1)
        kh1 = torch.empty_like(attn.k_h)
        rp1 = torch.empty_like(attn.row_ptr)
        ci1 = torch.empty_like(attn.col_idx)
        if kind != "ratio":
            pxa.pxa_budget_estimate_ex(cfg, full, dev["q"], dev["k"], S1, kh1,
                                       torch.empty_like(attn.masses), attn.ws[L.budget_ws:],
                                       ws_bytes=bws_bytes)
        pxa.pxa_block_select_ex(cfg, full, S1, None if kind == "ratio" else kh1, rp1, ci1,
                                attn.ws[L.select_ws:], ws_bytes=pxa.pxa_select_workspace_bytes(cfg))

        def dense_mask(rp_t, ci_t):
            rows = torch.repeat_interleave(torch.arange(H * nb, device="cuda"),
                                           (rp_t[1:] - rp_t[:-1]).long())
            m = torch.zeros(H * nb * nb, dtype=torch.bool, device="cuda")
            m[rows * nb + ci_t[: int(rp_t[-1])].long()] = True
            return m

        m_s, m_1 = dense_mask(attn.row_ptr, attn.col_idx), dense_mask(rp1, ci1)
        causal_total = H * nb * (nb + 1) // 2
        diff = int((m_s ^ m_1).sum())
        stride_cmp = {"causal_blocks_differing": diff,
                      "fraction_identical": round(1.0 - diff / causal_total, 5),
                      "kept_every_query": int(m_1.sum()), "kept_strided": int(m_s.sum()),
                      "kept_in_both": int((m_s & m_1).sum())}
        del S1, kh1, rp1, ci1, m_s, m_1
        log(f"strided mask vs every-query mask: {stride_cmp}")
    pool_bytes = (H + Hkv + 2 * G) * N * d * 2
    budget_bytes = Hkv * N * d * 2 + H * B * d * 2 + H * nb * B * 4 * 2
    select_bytes = G * nb * nb * 4 + H * nb * 4 * 3 + n_kept * 4

    # CPU oracle on a bounded sample (rank 0, one GPU)
    cpu = mask_vs_oracle = None
    if not a.no_cpu_baseline:
        ci = attn.col_idx.cpu().numpy()
        rng = np.random.default_rng(7)
        samp = []
        for h in sorted(rng.choice(H, size=min(H, 16), replace=False).tolist()):
            for I in rng.integers(nb // 4, nb, size=16).tolist():
                r = h * nb + I
                samp.append((h, I, ci[rp[r]:rp[r + 1]].astype(np.int64)))
        log("timing the CPU oracle on a sample")
        cpu, mask_vs_oracle = cpu_baseline(
            cfg, x, samp, n_kept, (rp, ci, kh if kind != "ratio" else None),
            budget_s=a.cpu_budget_s, last_blocks=budget.last_blocks, budget_kind=kind,
            score_stride=a.score_stride, gamma=gamma,
            budget_param=budget.fixed_blocks if kind == "fixed" else budget.ratio)
        cpu["value"] = round(cpu["value"], 1)
        log(f"mask vs the oracle's chain on sampled rows: {mask_vs_oracle}")

    res = {
        "metric": METRIC, "value": round(ms_step, 3), "unit": "ms", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generator, bf16, inputs resident in HBM)",
        "config": {"workload": f"{wl.name}: {wl.description}", "num_heads": H, "num_kv_heads": Hkv,
                   "head_dim": d, "seq_len": N, "block": B, "num_proxies": G, "gamma": gamma,
                   "batch": 1, "budget": budget_desc, "score_stride": a.score_stride,
                   "skip_threshold": a.skip_threshold,
                   "input_sha256_16": digest},
        "speedup_vs_dense": round(dense_ms / ms_step, 3),
        "dense_ms": round(dense_ms, 3),
        "torch_sdpa_dense": sdpa,
        "estimation_ms": round(est_ms, 3),
        "estimation_pct_of_dense": round(100.0 * est_ms / dense_ms, 3),
        "estimation_stages_standalone_ms": round(est_stages_ms, 3),
        "kept_density": round(density, 4),
        "mask_vs_every_query_scoring": stride_cmp,
        "mask_vs_oracle_sampled": mask_vs_oracle,
        "running_max_skip": skip_cmp,
        "k_h": kh.tolist() if kind != "ratio" else None,
        "stage_ms": {n: round(v, 4) for n, v in stage.items()},
        "kept_block_mfma_util": round(kept_tflops / PEAK_BF16_TFLOPS, 4),
        "dense_mfma_util": round(tflops(f_dense, dense_ms) / PEAK_BF16_TFLOPS, 4),
        "score_mfma_util": round(tflops(f_score, stage["score"]) / PEAK_BF16_TFLOPS, 4),
        "hbm_gbs": {"pool": round(pool_bytes / (stage["pool"] * 1e-3) / 1e9, 1),
                    "budget": round(budget_bytes / (stage["budget"] * 1e-3) / 1e9, 1),
                    "select": round(select_bytes / (stage["select"] * 1e-3) / 1e9, 1)},
        "roofline": {"kernel": "fa_prefill_kernel<128,sparse>", "bound": "mfma",
                     "achieved": round(kept_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kept_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
        "host_wall_ms_per_step": round(wall_ms, 3),
    }
    traffic, source = None, None
    if not a.no_live_traffic:
        traffic = live_traffic(a)
        source = "rocprofv3 FETCH_SIZE + WRITE_SIZE in this run" if traffic is not None else None
    if traffic is None:
        traffic = profiled_traffic(wl.name, res["config"])
        source = (f"profiles/fa_prefill_sparse_{wl.name}.md" if traffic is not None else None)
    res["roofline"]["traffic"] = round(traffic) if traffic is not None else None
    res["roofline"]["traffic_source"] = source
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
