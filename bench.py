"""Benchmark of one block-parallel speculative draft-and-verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C1] [--no-cpu-baseline]

A step = dflash_draft_step (n_new = S freshly committed rows appended onto
C - S cached rows, block of S) + markov_bias_sample (parallel sampling when the
workload has no Markov head) + spec_verify against synthetic target logits,
with every input already resident in HBM.  The context length is reset to
C - S before each step so each step does identical work.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import WORKLOADS, inputs  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0       # dense bf16 matrix-core peak (no sparsity)
METRIC = "draft-verify steps/sec + HBM GB/s, B=8 block=16 ctx=4K vocab=152K (1 GPU)"


def step_algorithmic_bytes(w, ab=None):
    """Bytes of one whole step: the drafter GEMMs, attention, the sequential head
    (its GEMM and logits update) or, without a head, the sampling pass, and verify.
    The per-group entries that are parts of these (weights alone, the head's GEMM)
    or flop counts are not added."""
    ab = algorithmic_bytes(w) if ab is None else ab
    return ab["gemm"] + ab["attention"] + ab["verify"] + (ab["markov"] if w.markov_rank > 0 else ab["sample"])


def algorithmic_bytes(w):
    """Bytes the step must move at minimum, per kernel group (see the design notes)."""
    es = 2 if w.dtype == "bf16" else 4
    B, S, G, C, L, H = w.batch, w.block, w.gamma, w.ctx, w.n_layers, w.hidden
    nq, nkv, d, F, V, nT, r = (w.n_q_heads, w.n_kv_heads, w.head_dim, w.mlp_dim, w.vocab,
                               w.n_target_layers, w.markov_rank)
    Mb, Mc = B * S, B * S
    per_layer_w = (nq * d * H + 2 * nkv * d * H + H * nq * d + 3 * F * H) * es
    gemm_w = L * per_layer_w + (H * nT * H + V * H) * es
    # activations in/out of every GEMM (X read once per launch, fp32 result written once;
    # the gate|up GEMM writes the bf16 SwiGLU product in its gated (bf16) form)
    gated = w.dtype == "bf16"
    gateup_out = Mb * F * es if gated else Mb * 2 * F * 4
    gemm_act = (Mc * nT * H * es + Mc * H * 4
                + L * ((Mc + Mb) * H * es + (Mc * 2 * nkv + Mb * (nq + 2 * nkv)) * d * 4
                       + Mb * nq * d * es + Mb * H * 4 + Mb * H * es + gateup_out
                       + Mb * F * es + Mb * H * 4)
                + B * G * H * es + B * G * V * 4)
    Ck = min(C, w.window) if w.window > 0 else C        # context keys a block row attends
    attn = L * (B * nkv * (Ck + S) * d * 2 * es + Mb * nq * d * es * 2)
    sample = B * G * V * 4                               # read final logits once
    markov = (V * r * es + B * G * V * 4 * 2) if r > 0 else 0
    verify = B * (G + 1) * V * 4 + 2 * B * V * 4        # target rows + the two rows at the rejection
    # dense products of the drafter GEMMs (the QKV GEMM runs over context and block rows;
    # the context rows need keys and values only)
    gemm_flops = 2.0 * (Mc * H * nT * H + B * G * V * H
                        + L * ((Mc * 2 * nkv + Mb * (nq + 2 * nkv)) * d * H + Mb * H * nq * d + Mb * 2 * F * H
                               + Mb * H * F))
    # the Markov head's per-position GEMM: W once, gathered U rows, logits rows read and written
    markov_gemm = (V * r * es + B * G * r * es + 2 * B * G * V * 4) if r > 0 else 0
    markov_flops = 2.0 * B * G * V * r
    return {"gemm": gemm_w + gemm_act, "gemm_weights": gemm_w, "gemm_flops": gemm_flops, "attention": attn,
            "sample": sample, "markov": markov, "markov_gemm": markov_gemm, "markov_flops": markov_flops,
            "verify": verify}


class Step:
    def __init__(self, w, seed=0, reuse=None, head="markov"):
        """reuse: another Step of a workload with the same drafter weights (block
        or Markov-head sweeps), whose host and device weights are shared.
        head: the sequential head, "markov" (the default head) or "rnn"."""
        import torch
        from block_speculative_decoding_amd import dfspec as D
        self.D, self.torch, self.w = D, torch, w
        dev = "cuda"
        t0 = time.time()

        def up(a, kind):
            a = np.ascontiguousarray(a)
            if kind == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        self.cfg = D.DrafterConfig.of(w)
        if reuse is not None:
            self.np_weights, self.wdev = reuse.np_weights, reuse.wdev   # the block is not part of them
        else:
            self.np_weights = inputs.drafter_weights(w, seed)
            # bf16 matrices in the tile-packed layout the matrix-core kernels stream (packed once here)
            self.wdev = D.DrafterWeights(self.cfg, {k: up(v, w.dtype) for k, v in self.np_weights.items()},
                                         packed=w.dtype == "bf16")
        step = inputs.step_inputs(w, seed)
        self.np_step = step
        kc, vc = inputs.cache_prefix(w, seed, step["ctx_len"])
        self.np_cache = (kc, vc)
        self.k, self.v = D.cache_from_logical(up(kc, w.dtype), up(vc, w.dtype))
        self.hidden = up(step["hidden_new"], w.dtype)
        self.n_new = up(step["n_new"], "i32")
        self.ctx0 = up(step["ctx_len"], "i32")
        self.ctx = self.ctx0.clone()
        self.last = up(step["last_token"], "i32")
        B, G, V = w.batch, w.gamma, w.vocab
        self.logits = torch.empty((B, G, V), dtype=torch.float32, device=dev)
        self.tokens = torch.empty((B, G), dtype=torch.int32, device=dev)
        self.row_stats = torch.empty((B, G, 2), dtype=torch.float64, device=dev)
        self.out = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
        self.nacc = torch.empty((B,), dtype=torch.int32, device=dev)
        ud, ua, uf = inputs.uniforms(w, seed)
        self.ud, self.ua, self.uf = up(ud, "f32"), up(ua, "f32"), up(uf, "f32")
        self.head = head if w.markov_rank > 0 else "markov"
        self.A = up(inputs.rnn_recurrence(w, seed), w.dtype) if self.head == "rnn" else None
        if w.markov_rank > 0:
            U, Wt = inputs.markov_factors(w, seed)
            self.U, self.Wt = up(U, w.dtype), up(Wt, w.dtype)
            self.wt_packed = w.dtype == "bf16"
            if self.wt_packed:
                self.Wt = D.pack_matrix(self.Wt.view(w.vocab, w.markov_rank))
        else:
            self.U = self.Wt = None
            self.wt_packed = False
        self.ws_d = torch.empty(D.dflash_draft_workspace_size(self.cfg, B, step["n_new_max"]),
                                dtype=torch.uint8, device=dev)
        self.ws_m = torch.empty(D.rnn_bias_sample_workspace_size(B, G, V, w.markov_rank) if self.head == "rnn"
                                else D.markov_bias_sample_workspace_size(B, G, V), dtype=torch.uint8, device=dev)
        self.ws_v = torch.empty(D.spec_verify_workspace_size(B, G, V), dtype=torch.uint8, device=dev)
        if w.target_noise_std > 0:       # target = draft logits + noise: needs one draft pass first
            self.draft()
            self.sample()
            torch.cuda.synchronize()
            self.target = up(inputs.target_logits(w, seed, draft_logits=self.logits.cpu().numpy()), "f32")
        else:
            self.target = up(inputs.target_logits(w, seed), "f32")
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0

    def draft(self):
        self.ctx.copy_(self.ctx0)
        self.D.dflash_draft_step(self.cfg, self.wdev, self.hidden, self.n_new, self.w.block, self.w.ctx,
                                 self.k, self.v, self.ctx, self.last, self.logits, self.ws_d)

    def sample(self):
        if self.head == "rnn":
            self.D.rnn_bias_sample(self.logits, self.U, self.Wt, self.A, self.last, self.ud, self.w.temperature,
                                   self.tokens, self.row_stats, self.ws_m, wt_packed=self.wt_packed)
            return
        self.D.markov_bias_sample(self.logits, self.U, self.Wt, self.last, self.ud, self.w.temperature,
                                  self.tokens, self.row_stats, self.ws_m, wt_packed=self.wt_packed)

    def verify(self):
        self.D.spec_verify(self.logits, self.target, self.tokens, self.ua, self.uf, self.w.temperature,
                           self.row_stats, self.out, self.nacc, self.ws_v)

    def __call__(self):
        self.draft()
        self.sample()
        self.verify()


def time_steps(step, K):
    torch = step.torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(K):
        step()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / K


def achievable_peaks(torch):
    """Measured reference peaks of this GPU, for fractions beside the datasheet's:
    a plain 1 GiB device copy (bytes read + written per second) and a large
    square bf16 library GEMM (torch.mm, 8192^3, contiguous operands)."""
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    c = torch.empty(8192, 8192, dtype=torch.bfloat16, device="cuda")
    out = {}
    for name, fn, units in (("copy_gbps", lambda: dst.copy_(src), 2.0 * src.numel() * 4 / 1e9),
                            ("gemm_tflops", lambda: torch.mm(a, b, out=c), 2.0 * 8192 ** 3 / 1e12)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = units / (e0.elapsed_time(e1) / 10 * 1e-3)
    del src, dst, a, b, c
    torch.cuda.empty_cache()
    return out


def profile_group(step, group, K, launches_per_step):
    D = step.D
    D.dfs_profile_begin(group, K * launches_per_step + 8)
    ms = time_steps(step, K)
    n, tot = D.dfs_profile_end()
    return n, tot, ms


def cpu_baseline(w, step, max_rows=8):
    """The oracle, as it stands, on one step of the same workload: one drafter call
    (the append and the block of every sampled batch row in one call), their
    sampling and their verification, timed once.  Up to `max_rows` batch rows
    (all 8 at the metric's configuration, so the whole step); for larger batches
    the first `max_rows` rows, scaled to the batch."""
    import oracle
    from oracle import drafter as od
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    n = min(w.batch, max_rows)
    rows = slice(0, n)
    kc, vc = step.np_cache
    st = step.np_step
    ko = kc[:, rows].copy()
    vo = vc[:, rows].copy()
    ud, ua, uf = (x[rows] for x in inputs.uniforms(w, 0))
    tgt = step.target[rows].cpu().numpy()
    if w.markov_rank > 0:
        U, Wt = inputs.markov_factors(w, 0)
    t0 = time.perf_counter()
    base, _ = od.draft_step(od.DrafterShape.of(w.with_(batch=n)), step.np_weights, st["hidden_new"][rows],
                            st["n_new"][rows], ko, vo, st["ctx_len"][rows], st["last_token"][rows])
    if w.markov_rank > 0 and step.head == "rnn":
        final, tok, _, _ = oracle.rnn_sample(base, U, Wt, inputs.rnn_recurrence(w, 0), w.dtype, st["last_token"][rows],
                                             ud, w.temperature)
    elif w.markov_rank > 0:
        final, tok, _ = oracle.markov_sample(base, U, Wt, w.dtype, st["last_token"][rows], ud, w.temperature)
    else:
        final, tok, _ = oracle.markov_sample(base, None, None, w.dtype, st["last_token"][rows], ud, w.temperature)
    oracle.verify(final, tgt, tok, ua, uf, w.temperature)
    secs = time.perf_counter() - t0
    whole = n == w.batch
    return {"value": (n / w.batch) / secs, "unit": "steps/s", "cores": blas_threads or 1, "kind": "oracle",
            "host_cores_visible": cores, "blas_threads": blas_threads,
            "sample": (f"one whole step (all {n} batch rows in one oracle call: drafter incl. its {w.block}-row "
                       f"append, sampling, verify), {secs:.1f} s" if whole else
                       f"batch rows 0..{n - 1} of {w.batch} in one oracle call ({secs:.1f} s), scaled x{w.batch / n:g}")}


# ---------------------------------------------------------------- rocprofv3 summaries

GEMM_SOURCES = ["block_speculative_decoding_amd/csrc/gemm.hip", "block_speculative_decoding_amd/csrc/kernels.h",
                "block_speculative_decoding_amd/csrc/common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_stream_C1_hbm_traffic.txt")


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per GEMM launch recorded with the PMC counters, if the GEMM
    sources still hash to the value recorded next to them (else None)."""
    try:
        kv = dict(l.split(":", 1) for l in open(TRAFFIC_FILE).read().splitlines() if ":" in l and not l.startswith(" "))
        if kv.get("source_sha256", "").strip() != gemm_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _short(name):
    import re
    return re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", "").replace("void ", ""))


def summarize_rocprof(d, steps):
    """Print the per-kernel table of a rocprofv3 --stats run, or the per-kernel
    average counters of a --pmc run, found under directory d."""
    import csv
    import glob
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    pmc = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if stats:
        rows = list(csv.DictReader(open(stats[0])))
        print(f"{'kernel':60s} {'calls':>6s} {'calls/step':>10s} {'total us':>10s} {'avg us':>8s} {'us/step':>8s}")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            n, tot = int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3
            print(f"{_short(r['Name'])[:60]:60s} {n:6d} {n / steps:10.2f} {tot:10.1f} {tot / n:8.2f} {tot / steps:8.1f}")
    for f in pmc:
        agg = {}
        for r in csv.DictReader(open(f)):
            k = (_short(r["Kernel_Name"])[:60], r["Counter_Name"])
            a = agg.setdefault(k, [0, 0.0])
            a[0] += 1
            a[1] += float(r["Counter_Value"])
        print(f"{'kernel':60s} {'counter':12s} {'dispatches':>10s} {'avg/dispatch':>17s}")
        for (k, c), (n, v) in sorted(agg.items(), key=lambda x: -x[1][1]):
            print(f"{k:60s} {c:12s} {n:10d} {v / n:17.1f}")


def _pmc_agg(d):
    """Per-kernel (dispatches, sum) of each counter in a rocprofv3 --pmc run."""
    import csv
    import glob
    agg = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            k = (_short(r["Kernel_Name"]), r["Counter_Name"])
            a = agg.setdefault(k, [0, 0.0])
            a[0] += 1
            a[1] += float(r["Counter_Value"])
    return agg


def _pmc_avg(d):
    """Per-kernel average of each counter (per dispatch) in a rocprofv3 --pmc run."""
    return {k: v / n for k, (n, v) in _pmc_agg(d).items()}


def _copy_scales(cal_fetch_dir, cal_write_dir):
    """Bytes per KiB of FETCH_SIZE and of WRITE_SIZE, from what a plain 1 GiB device
    copy (bench.py --calibrate-copy) reads on those counters."""
    copy_bytes = float(1 << 30)
    f_cal = [v for (k, c), v in _pmc_avg(cal_fetch_dir).items() if "copy" in k.lower() and c == "FETCH_SIZE"]
    w_cal = [v for (k, c), v in _pmc_avg(cal_write_dir).items() if "copy" in k.lower() and c == "WRITE_SIZE"]
    return copy_bytes / (max(f_cal) * 1024.0), copy_bytes / (max(w_cal) * 1024.0), max(f_cal), max(w_cal)


def record_gemm_traffic(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, workload, commands):
    """Write the HBM bytes per drafter GEMM launch (all dfs::gemm_* dispatches of a
    --pmc run, copy-calibrated) with the hash of the GEMM sources, the figure the
    benchmark reports as roofline.traffic while the sources are unchanged."""
    f_scale, w_scale, f_cal, w_cal = _copy_scales(cal_fetch_dir, cal_write_dir)
    fa, wa = _pmc_agg(fetch_dir), _pmc_agg(write_dir)
    rows, n_all, bytes_all = [], 0, 0.0
    for (k, c), (n, v) in sorted(fa.items()):
        if c != "FETCH_SIZE" or not k.startswith("dfs::gemm_"):
            continue
        wn, wv = wa.get((k, "WRITE_SIZE"), (n, 0.0))
        per = (v / n) * 1024.0 * f_scale + (wv / wn) * 1024.0 * w_scale
        rows.append((k, n, v / n, wv / wn, per))
        n_all += n
        bytes_all += n * per
    w = WORKLOADS[workload]
    alg = algorithmic_bytes(w)["gemm"] / (4 * w.n_layers + 2)
    out = [f"HBM traffic of the drafter GEMM launches, {workload} workload ({w.name}), one MI355X.", "",
           "Commands (run from the repository root on the GPU machine):"] + [f"  {c}" for c in commands] + [
        "", f"Calibration: a plain 1 GiB device copy reads FETCH_SIZE = {f_cal:.1f} KiB and WRITE_SIZE = {w_cal:.1f} KiB",
        f"per dispatch, so bytes fetched = {f_scale:.3f} x FETCH_SIZE KiB x 1024 and written = {w_scale:.3f} x WRITE_SIZE.",
        "", f"  {'kernel':56s} {'dispatches':>10s} {'FETCH KiB':>10s} {'WRITE KiB':>10s} {'bytes/dispatch':>15s}"]
    out += [f"  {k[:56]:56s} {n:10d} {f:10.1f} {wr:10.1f} {per:15.0f}" for k, n, f, wr, per in rows]
    out += ["", f"Average HBM bytes per GEMM launch = {bytes_all / n_all:.0f}",
            f"Algorithmic bytes per launch (weights once + activations in/out) = {alg:.0f}",
            f"Ratio traffic / algorithmic = {bytes_all / n_all / alg:.3f}", "",
            f"traffic_bytes_per_launch: {bytes_all / n_all:.0f}", f"source_sha256: {gemm_source_hash()}", "",
            "(bench.py reports this traffic only while the GEMM sources hash to source_sha256.)"]
    open(TRAFFIC_FILE, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def summarize_traffic(stats_dir, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, steps):
    """Per-kernel HBM traffic of a workload step: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, from two --pmc runs) scaled by what the same counters read for a plain
    1 GiB device copy (bench.py --calibrate-copy), against each kernel's average
    duration from a --kernel-trace --stats run: bytes per dispatch / duration.
    steps: the steps (timed + warm-up) of the --kernel-trace --stats run, for calls
    per step."""
    import csv
    import glob
    f_scale, w_scale, f_cal, w_cal = _copy_scales(cal_fetch_dir, cal_write_dir)
    print(f"calibration: a 1 GiB device copy reads FETCH_SIZE {f_cal:.1f} KiB and WRITE_SIZE {w_cal:.1f} KiB "
          f"per dispatch -> bytes read = {f_scale:.3f} x FETCH_SIZE KiB x 1024, written = {w_scale:.3f} x WRITE_SIZE")
    fetch, write = _pmc_avg(fetch_dir), _pmc_avg(write_dir)
    rows = list(csv.DictReader(open(glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)[0])))
    print(f"{'kernel':58s} {'calls/step':>10s} {'avg us':>8s} {'read MB':>9s} {'write MB':>9s} {'GB/s':>8s} {'of 8 TB/s':>9s}")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = _short(r["Name"])
        n, avg_us = int(r["Calls"]), float(r["AverageNs"]) / 1e3
        fk, wk = fetch.get((name, "FETCH_SIZE")), write.get((name, "WRITE_SIZE"))
        if fk is None or wk is None or n / steps < 0.99 or not name.startswith("dfs::"):
            continue
        rb, wb = fk * 1024.0 * f_scale, wk * 1024.0 * w_scale
        gbps = (rb + wb) / (avg_us * 1e-6) / 1e9
        print(f"{name[:58]:58s} {n / steps:10.2f} {avg_us:8.2f} {rb / 1e6:9.2f} {wb / 1e6:9.2f} {gbps:8.0f} "
              f"{gbps / HBM_PEAK_GBPS:9.3f}")


def sweeps(steps, warmup):
    """Secondary measurements: draft time vs block size (the block drafter's cost
    should be nearly flat in the block size) and the Markov head's share of the
    step at draft lengths 4 and 16 (the pages quote a 0.2-1.3 % latency cost for
    going from 4 to 16 draft tokens).  One JSON line per point."""
    base = None
    for S in (4, 8, 16, 32):
        w = WORKLOADS["C1"].with_(name=f"dflash_bf16_b8_s{S}_c4096_v151936", block=S)
        st = Step(w, reuse=base)
        base = base or st
        for _ in range(warmup):
            st()
        ms = time_steps(st, steps)
        n, tot, _ = profile_group(st, "gemm", steps, 64)
        print(json.dumps({"sweep": "block", "workload": w.name, "block": S, "gamma": S - 1,
                          "ms_per_step": ms, "gemm_ms_per_step": tot / steps}), flush=True)
    base = None
    for S in (5, 17):   # draft lengths 4 and 16
        w = WORKLOADS["C2"].with_(name=f"dspark_markov_bf16_b32_s{S}_c4096_v129280", block=S)
        st = Step(w, reuse=base)
        base = base or st
        for _ in range(warmup):
            st()
        ms = time_steps(st, steps)
        n, tot, _ = profile_group(st, "markov", steps, 64 * S)
        print(json.dumps({"sweep": "markov", "workload": w.name, "gamma": S - 1, "ms_per_step": ms,
                          "markov_ms_per_step": tot / steps, "markov_share": tot / steps / ms}), flush=True)


def sps_profile(wl, steps=10, warmup=2, seed=0):
    """The throughput curve the prefix scheduler uses, measured once at startup:
    this library's whole step (draft + sample + verify) at batch sizes 1, 2, 4, ...
    up to the workload's, as verify passes per second against the rows verified
    (batch x block)."""
    w0 = WORKLOADS[wl]
    batches = [b for b in (1, 2, 4, 8, 16, 32, 64, 128) if b < w0.batch] + [w0.batch]
    rows, sps = [], []
    base = None
    for b in batches:
        w = w0.with_(name=f"{w0.name}_sps_b{b}", batch=b)
        st = Step(w, seed=seed, reuse=base)
        for _ in range(warmup):
            st()
        ms = time_steps(st, steps)
        rows.append(b * w.block)
        sps.append(1000.0 / ms)
        if base is None:
            base = st
        else:
            del st
    return rows, sps


def loop_bench(wl, K, R, sigma=1.0, seed=0, schedule=False):
    """On-device multi-step loop: K cycles of draft -> sample -> [synthetic target]
    -> verify -> advance captured into one HIP graph and replayed R times, the
    accepted count of each cycle driving the next append on the device.  Targets
    are the final draft rows plus N(0, sigma^2) noise, the bonus row N(0, 3^2),
    so acceptance is partial.  Reports time per cycle (graph and eager), the
    synthetic-target time alone, the mean tokens committed per cycle (tau) and
    L = (cycle time without the synthetic target) / tau.  With ``schedule`` the
    prefix scheduler sets each request's verify length every cycle from seeded
    survival scores (standing in for a confidence head) and the SPS curve of
    this library's step profiled first.  One JSON line."""
    import torch
    from block_speculative_decoding_amd import dfspec as D
    from block_speculative_decoding_amd.loop import SpecLoop
    w0 = WORKLOADS[wl]
    B, S, G, V = w0.batch, w0.block, w0.gamma, w0.vocab
    total = K * (R + 2)                      # eager warm-up, eager timed, R graph replays
    w = w0.with_(ctx=w0.ctx + total * S + 64)   # cache capacity for every cycle's append
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(a, kind):
        a = np.ascontiguousarray(a)
        if kind == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    cfg = D.DrafterConfig.of(w)
    np_w = inputs.drafter_weights(w0, seed)
    wdev = D.DrafterWeights(cfg, {k: up(v, w.dtype) for k, v in np_w.items()}, packed=w.dtype == "bf16")
    del np_w
    L, nkv, d, M = w.n_layers, w.n_kv_heads, w.head_dim, w.max_ctx
    # cache contents below the starting context (device-generated; their values do not matter here)
    kl = (torch.randn((L, B, M, nkv, d), generator=gen, device=dev) * 1.28).to(tdt)
    vl = (torch.randn((L, B, M, nkv, d), generator=gen, device=dev) * 1.28).to(tdt)
    k, v = D.cache_from_logical(kl, vl)
    del kl, vl
    ctx0 = torch.full((B,), w0.ctx - S, dtype=torch.int32, device=dev)
    last0 = torch.randint(0, V - 1, (B,), generator=gen, device=dev, dtype=torch.int32)
    n0 = torch.full((B,), S, dtype=torch.int32, device=dev)
    U = Wt = None
    packed = False
    if w.markov_rank > 0:
        Un, Wn = inputs.markov_factors(w0, seed)
        U, Wt = up(Un, w.dtype).view(V, w.markov_rank), up(Wn, w.dtype).view(V, w.markov_rank)
        packed = w.dtype == "bf16"
        if packed:
            Wt = D.pack_matrix(Wt)
    curve = sps_profile(wl, seed=seed) if schedule else None
    lp = SpecLoop(cfg, wdev, k, v, ctx0, last0, n0, w.temperature, U, Wt, wt_packed=packed, curve=curve)
    nT_H = w.n_target_layers * w.hidden
    pool = [dict(h=torch.randn((B, S, nT_H), generator=gen, device=dev).to(tdt),
                 ud=torch.rand((B, G), generator=gen, device=dev) * 0.999999,
                 ua=torch.rand((B, G), generator=gen, device=dev) * 0.999999,
                 uf=torch.rand((B,), generator=gen, device=dev) * 0.999999,
                 nz=torch.randn((B, S, V), generator=gen, device=dev),
                 sv=torch.rand((B, G), generator=gen, device=dev)) for _ in range(K)]
    for p_ in pool:
        p_["nz"][:, :G].mul_(sigma)
        p_["nz"][:, G].mul_(3.0)

    def target_fn(nz):
        def f(final, target):
            target[:, :G].copy_(final)
            target[:, :G].add_(nz[:, :G])
            target[:, G].copy_(nz[:, G])
        return f

    def run():
        for p_ in pool:
            lp.cycle(p_["h"], p_["ud"], p_["ua"], p_["uf"], target_fn(p_["nz"]), survival=p_["sv"] if schedule else None)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    run()                                     # eager warm-up
    torch.cuda.synchronize()
    ev[0].record()
    run()
    ev[1].record()
    torch.cuda.synchronize()
    eager_ms = ev[0].elapsed_time(ev[1]) / K
    ev[0].record()
    for p_ in pool:
        target_fn(p_["nz"])(lp.logits, lp.target)
    ev[1].record()
    torch.cuda.synchronize()
    synth_ms = ev[0].elapsed_time(ev[1]) / K
    sched_us = None
    if schedule:
        ev[0].record()
        for p_ in pool:
            D.spec_schedule_verify(p_["sv"], curve[0], curve[1], lp.n_verify)
        ev[1].record()
        torch.cuda.synchronize()
        sched_us = ev[0].elapsed_time(ev[1]) / K * 1e3
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            run()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    lp.tau_sum.zero_()
    ev[0].record()
    for _ in range(R):
        g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    graph_ms = ev[0].elapsed_time(ev[1]) / (K * R)
    tau = float(lp.tau_sum.double().sum().item()) / (B * K * R)
    core_ms = graph_ms - synth_ms
    print(json.dumps({"loop": w0.name, "cycles": K * R, "cycles_per_graph": K, "graph": True,
                      "ms_per_cycle": graph_ms, "ms_per_cycle_eager": eager_ms,
                      "target_synthesis_ms": synth_ms, "mean_tau": tau, "acceptance_rate": (tau - 1.0) / G,
                      "L_ms_per_token": core_ms / tau, "tokens_per_s": B * tau / (core_ms * 1e-3),
                      "target": f"final draft logits + N(0, {sigma}^2), bonus row N(0, 3^2)",
                      "final_ctx_len_max": int(lp.ctx_len.max().item()),
                      **({"schedule": {"curve_rows": curve[0], "curve_steps_per_s": [round(x, 1) for x in curve[1]],
                                       "mean_verify_length_last_cycle": float(lp.n_verify.double().mean().item()),
                                       "scheduler_kernel_us": sched_us}} if schedule else {})}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C1", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (reference for HBM byte counters)")
    ap.add_argument("--loop", action="store_true",
                    help="on-device multi-step loop: cycles captured in a HIP graph, tau and L (JSON line)")
    ap.add_argument("--loop-cycles", type=int, default=8, help="cycles per captured graph")
    ap.add_argument("--schedule", action="store_true",
                    help="with --loop: per-request verify lengths from the prefix scheduler (SPS profiled first)")
    ap.add_argument("--loop-replays", type=int, default=8, help="graph replays timed")
    ap.add_argument("--sweep", action="store_true",
                    help="secondary measurements: block-size and Markov draft-length sweeps (JSON line per point)")
    ap.add_argument("--head", default="markov", choices=("markov", "rnn"),
                    help="sequential head of workloads that have one (rnn: the optional RNN head)")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="print the kernel table / counter averages of a rocprofv3 output directory and exit")
    ap.add_argument("--record-gemm-traffic", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="write the GEMM launches' HBM bytes per launch (copy-calibrated FETCH/WRITE_SIZE runs of "
                         "--workload) with the GEMM sources' hash to the profiles record, and exit")
    ap.add_argument("--summarize-traffic", nargs=5, metavar=("STATS", "FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="per-kernel HBM traffic (copy-calibrated FETCH/WRITE_SIZE) against kernel durations, and exit")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.steps + args.warmup)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.steps + args.warmup)
        return
    if args.record_gemm_traffic:
        fd, wd, cf, cw = args.record_gemm_traffic
        run = f"--workload {args.workload} --steps {args.steps} --warmup {args.warmup} --no-cpu-baseline --no-roofline"
        record_gemm_traffic(fd, wd, cf, cw, args.workload, [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fd} -o p -- python bench.py {run}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {wd} -o p -- python bench.py {run}",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {cf} -o p -- python bench.py --calibrate-copy",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {cw} -o p -- python bench.py --calibrate-copy",
            f"python bench.py --record-gemm-traffic {fd} {wd} {cf} {cw} --workload {args.workload} "
            f"--steps {args.steps} --warmup {args.warmup}"])
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.sweep:
        sweeps(args.steps, args.warmup)
        return
    if args.loop:
        loop_bench(args.workload, args.loop_cycles, args.loop_replays, schedule=args.schedule)
        return
    if args.calibrate_copy:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": src.numel() * 4, "launches": 5}))
        return
    w = WORKLOADS[args.workload]
    print(f"[bench] setting up {w.name}", file=sys.stderr, flush=True)
    step = Step(w, head=args.head)
    print(f"[bench] setup {step.setup_s:.1f}s; warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    ms = time_steps(step, args.steps)
    print(f"[bench] {ms:.3f} ms/step", file=sys.stderr, flush=True)
    ab = algorithmic_bytes(w)
    step_bytes = step_algorithmic_bytes(w, ab)
    res = {
        "metric": METRIC, "value": 1000.0 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded; weights N(0,0.02^2))",
        "config": {"workload": w.name, "batch": w.batch, "block": w.block, "ctx": w.ctx, "vocab": w.vocab,
                   "drafter_layers": w.n_layers, "hidden": w.hidden, "markov_rank": w.markov_rank,
                   **({"head": "rnn"} if step.head == "rnn" else {})},
        "hbm_gbps": step_bytes / (ms * 1e-3) / 1e9,
        "hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
    }
    if not args.no_roofline:
        L = w.n_layers
        # GEMM launches of one step: fc, 4 per layer, LM head; a sequential head whose
        # product runs through the plain GEMM launcher adds one per drafted position
        # (the fused rank-256 Markov product is timed with the head instead)
        per_step = 4 * L + 2 + (w.gamma if w.markov_rank > 0 else 0)
        n, tot, ms_p = profile_group(step, "gemm", args.steps, per_step)
        per_launch_ms = tot / max(n, 1)
        launches_per_step = n / args.steps
        head_in_group = launches_per_step > 4 * L + 2 + 0.5
        step_bytes_g = ab["gemm"] + (ab["markov_gemm"] if head_in_group else 0)
        step_flops_g = ab["gemm_flops"] + (ab["markov_flops"] if head_in_group else 0)
        bytes_per_launch = step_bytes_g / launches_per_step
        flops_per_launch = step_flops_g / launches_per_step
        kernel = "drafter GEMM launches (gemm_stream_bf16" + (", gemm_tile_bf16" if w.batch * w.block > 256 else "") \
            + (", Markov-head GEMMs" if head_in_group else "") + ")"
        ach = achievable_peaks(step.torch)
        if w.batch * w.block > 256 and w.dtype == "bf16":
            # M > 256: the drafter GEMMs are bound by the matrix cores
            achieved = flops_per_launch / (per_launch_ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                    "achievable_peak": ach["gemm_tflops"], "achievable_peak_source": "torch.mm bf16 8192^3",
                    "frac_of_achievable": achieved / ach["gemm_tflops"]}
        else:
            achieved = bytes_per_launch / (per_launch_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBPS,
                    "traffic": recorded_traffic() if w.name == WORKLOADS["C1"].name else None,
                    "achievable_peak": ach["copy_gbps"], "achievable_peak_source": "1 GiB device copy",
                    "frac_of_achievable": achieved / ach["copy_gbps"]}
        res["roofline"] = {"kernel": kernel, **roof, "algorithmic_bytes_per_launch": bytes_per_launch,
                           "flops_per_launch": flops_per_launch, "launches_per_step": launches_per_step,
                           "avg_launch_us": per_launch_ms * 1e3, "gemm_ms_per_step": tot / args.steps,
                           "ms_per_step_profiled": ms_p}
        groups = {}
        for g, per_step in (("attention", L), ("verify", 1), ("sample", 1), ("markov", 1), ("elementwise", 0)):
            if g == "markov" and w.markov_rank == 0:
                continue
            if g == "sample" and w.markov_rank > 0:
                continue
            n, tot, _ = profile_group(step, g, args.steps, max(per_step, 1) * 64)
            t = tot / args.steps
            groups[g] = {"ms_per_step": t}
            if g in ab and ab[g] and t > 0:
                groups[g]["gbps"] = ab[g] / (t * 1e-3) / 1e9
                groups[g]["frac"] = groups[g]["gbps"] / HBM_PEAK_GBPS
        res["groups"] = groups
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, step)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
