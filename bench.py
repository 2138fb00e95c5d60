"""Benchmark: response tokens/s for logprob + entropy on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs logits,grpo,...]

Prints ONE JSON line. `value` is the throughput of the logits-in path on its
Qwen3-scale workload (4096 rows x 151936 vocabulary, bf16 logits, T=0.7,
top-p=0.95; rows = response tokens), with inputs resident in HBM, over
calls timed back to back between two HIP events on the launch stream.
`roofline` is that kernel's achieved HBM bandwidth (algorithmic bytes per
launch / launch time, the call being one launch) against 8 TB/s.
`cpu_baseline` is the fp64 oracle over all rows of the same workload on the
host's cores (one worker process per core, up to 16), timed before the GPU
is first used. Other built paths are reported under `legs`, each with the
same figures, the per-call mean, median and min from a second run with
events around every call (which adds the events' own cost to each), and the
GPU clock level sampled during its timed region.
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

METRIC = "response tokens/s for logprob+entropy (V=151936,H=4096) + % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6          # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk


def _profile_traffic(name):
    """HBM bytes per launch from the committed counter summary profiles/<name>.md,
    or None when that summary is missing or the kernel's sources have changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "|", "#")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in fields["source_files"].split():
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest()[:16] != fields["source_sha256_16"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def _spin_up(torch, fn, seconds=0.3):
    """Run the leg's own call for a moment (at least once) so that the timed
    steps see the clocks the power manager settles on for this workload, not
    the ramp out of idle while inputs were generated on the host nor the
    state another workload left behind."""
    t0 = time.perf_counter()
    while True:
        fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break


def _sclk_files():
    import glob
    return sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))


def _read_sclk(files):
    """The current shader clock (MHz) from the driver's DPM table (the line
    marked '*'), or None."""
    import re
    for f in files:
        try:
            for line in open(f):
                if "*" in line:
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                    if m:
                        return int(m.group(1))
        except OSError:
            continue
    return None


class _ClockSampler:
    """Samples the shader clock's DPM level every ~2 ms on a host thread while
    the timed calls run (it reads the driver's sysfs table only: no GPU work;
    the thread sleeps, and reads, without holding the interpreter lock)."""

    def __init__(self):
        import threading
        self.files = _sclk_files()
        self.samples = []
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self.stop.is_set():
            v = _read_sclk(self.files)
            if v is not None:
                self.samples.append(v)
            self.stop.wait(0.002)

    def __enter__(self):
        if self.files:
            self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        if self.files:
            self.thread.join()

    def summary(self):
        if not self.samples:
            return None
        return {"median_mhz": int(np.median(self.samples)), "min_mhz": int(min(self.samples)),
                "max_mhz": int(max(self.samples)), "samples": len(self.samples),
                "source": "pp_dpm_sclk current DPM level (the power manager's level, not a "
                          "kernel clock), sampled every ~2 ms"}


def _profiler_attached():
    """True under rocprofv3, whose preloaded library initialises the GPU before
    this program starts: no worker process may then be forked."""
    pre = os.environ.get("LD_PRELOAD", "")
    return "rocprof" in pre or any(k.startswith("ROCPROF") for k in os.environ)


_LAST_CLOCK = [None]


def _events_time(torch, fn, steps, warmup):
    """Timing of `fn` with HIP events on the current stream: the total ms of
    `steps` calls back to back between two events (the whole-job figure,
    nothing recorded between the calls), then the mean, min and median ms
    per call from `steps` more calls, each between its own pair of events.
    Returns (mean, total, min, median); the shader clock sampled during the
    back-to-back calls is left in _LAST_CLOCK."""
    _spin_up(torch, fn)
    for _ in range(warmup):
        fn()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with _ClockSampler() as clk:
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
    _LAST_CLOCK[0] = clk.summary()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return (float(np.mean(per)), float(t0.elapsed_time(t1)), float(np.min(per)),
            float(np.median(per)))


def _outs(torch, o):
    """The tensors of a call's result (dict, tuple or tensor), in a fixed order."""
    if isinstance(o, dict):
        return [o[k] for k in sorted(o) if torch.is_tensor(o[k])]
    if isinstance(o, (tuple, list)):
        return [t for t in o if torch.is_tensor(t)]
    return [o]


def _same(torch, a, b):
    """Bitwise equality (NaN-safe: the raw bytes are compared)."""
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    return torch.equal(a.contiguous().view(-1).view(torch.uint8),
                       b.contiguous().view(-1).view(torch.uint8))


_CHECK_DETERMINISM = [True]


def _determinism(torch, run_full, run_rows=None, n=0, seed=0, device="cuda:0"):
    """Outside the timed region: three calls on the same inputs must agree
    bitwise; with `run_rows(idx)` (the per-row outputs for the rows idx, in
    that order), the full batch's per-row outputs must equal, bitwise, those
    of 4 random contiguous splits of the rows (each piece its own call) and
    of one random permutation. Skipped with --no-determinism (for profiler
    runs, whose per-kernel averages should cover the timed calls only)."""
    if not _CHECK_DETERMINISM[0]:
        return {"skipped": "--no-determinism"}
    ref = [t.clone() for t in _outs(torch, run_full())]
    ok = True
    for _ in range(2):
        ok = all(_same(torch, a, b) for a, b in zip(ref, _outs(torch, run_full()))) and ok
    res = {"run_to_run_x3": "pass" if ok else "FAIL"}
    if run_rows is not None:
        g = torch.Generator().manual_seed(seed)
        full_rows = [t.clone() for t in run_rows(torch.arange(n, device=device))]
        ok = True
        for _ in range(4):
            cuts = sorted(set(torch.randint(1, n, (3,), generator=g).tolist()))
            bounds = [0] + cuts + [n]
            for a, b in zip(bounds[:-1], bounds[1:]):
                part = run_rows(torch.arange(a, b, device=device))
                ok = all(_same(torch, p, r[a:b]) for p, r in zip(part, full_rows)) and ok
        perm = torch.randperm(n, generator=g).to(device)
        part = run_rows(perm)
        ok = all(_same(torch, p, r[perm]) for p, r in zip(part, full_rows)) and ok
        res["batch_invariance_4splits_1perm"] = "pass" if ok else "FAIL"
    if torch.device(device).type == "cuda":
        torch.cuda.synchronize()
    return res


_CPU_ORACLE = [True]


def _cpu_oracle(fn, units, sample, blas=False):
    """The fp64 oracle timed on a bounded sample of the leg's workload on the
    host, as a baseline beside the GPU figure: with `blas`, its fp64 matrix
    products use every host core (BLAS threads = _cores()); otherwise one
    thread (per-row numpy work). Input widening and other preparation stay
    outside the timing."""
    if not _CPU_ORACLE[0]:
        return None
    try:
        from threadpoolctl import threadpool_limits
        n = _cores() if blas else 1
        with threadpool_limits(n):
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
        how = f"{n} BLAS threads" if blas else "one thread"
        return {"value": units / dt, "unit": "tokens/s", "cores": n, "kind": "oracle",
                "sample": f"{sample}, fp64 numpy, {how}, {dt:.2f}s"}
    except Exception as e:  # noqa: BLE001 -- the GPU figure stands without it
        return {"error": f"{type(e).__name__}: {e}"}


def _cores():
    """Host cores this process may use, capped at 16 (one GPU's share of a 128-core, 8-GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


_POOL = {}    # kind -> fn(lo, hi): oracle work on rows lo..hi (set before the pool forks)
_DATA = {}    # inputs generated for the CPU baselines, reused by the GPU legs
_CPU_BASE = {}


def _pool_task(task):
    kind, lo, hi = task
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        _POOL[kind](lo, hi)
    return hi - lo


def _pool_ready(_):
    return 0


def _parallel_oracle(kind, n, cores, chunk):
    """Wall seconds for the oracle over rows 0..n in `chunk`-row tasks on
    `cores` forked worker processes (one BLAS thread each). Called before the
    GPU is first used, so no worker inherits a GPU context."""
    import multiprocessing as mp
    tasks = [(kind, lo, min(lo + chunk, n)) for lo in range(0, n, chunk)]
    with mp.get_context("fork").Pool(cores) as pool:
        pool.map(_pool_ready, range(cores))          # workers started before the clock
        t0 = time.perf_counter()
        done = sum(pool.map(_pool_task, tasks, chunksize=1))
        dt = time.perf_counter() - t0
    assert done == n
    return dt


def cpu_baselines(synth):
    """The fp64 oracle on the host's cores, before any GPU call: every row of
    the logits-in workloads (4096 x 151936 bf16 and 256 x 8192 fp32) and the
    GRPO loss stage over every token of the packed batch. Inputs are
    generated first (untimed) and kept for the GPU legs."""
    from oracle import grpo as OG
    from oracle import logprob as OL
    cores = _cores()
    w = synth.workload("qwen")
    t_gen = time.perf_counter()
    arr = synth.logits_rows(w, range(w.N))
    y = synth.peak_targets(w, range(w.N))
    _DATA["qwen"] = (arr, y)
    Tq, pq = OL.f32(w.temperature), OL.f32(w.top_p)
    _POOL["qwen"] = lambda lo, hi: OL.logprob_from_logits(OL.widen_bf16(arr[lo:hi]), y[lo:hi],
                                                          Tq, pq)
    wt = synth.workload("tiny")
    arr_t = synth.logits_rows(wt, range(wt.N))
    y_t = np.argmax(arr_t, axis=1).astype(np.int64)
    _DATA["tiny"] = (arr_t, y_t)
    Tt, pt = OL.f32(wt.temperature), OL.f32(wt.top_p)
    _POOL["tiny"] = lambda lo, hi: OL.logprob_from_logits(arr_t[lo:hi].astype(np.float64),
                                                          y_t[lo:hi], Tt, pt)
    print(f"[bench] CPU baselines: inputs generated in {time.perf_counter() - t_gen:.1f}s; "
          f"{cores} worker processes", file=sys.stderr, flush=True)
    dt = _parallel_oracle("qwen", w.N, cores, 16)
    _CPU_BASE["logits"] = {"value": w.N / dt, "unit": "tokens/s", "cores": cores,
                           "kind": "oracle",
                           "sample": f"all {w.N} rows of the workload, fp64 numpy oracle "
                                     f"(sort-based nucleus per row), {cores} worker processes "
                                     f"x 1 thread, {dt:.1f}s wall"}
    dt = _parallel_oracle("tiny", wt.N, cores, 8)
    _CPU_BASE["tiny"] = {"value": wt.N / dt, "unit": "tokens/s", "cores": cores,
                         "kind": "oracle",
                         "sample": f"all {wt.N} rows, fp64 numpy oracle, {cores} worker "
                                   f"processes x 1 thread, {dt:.2f}s wall"}
    # the GRPO loss stage: one vectorised call over the whole packed batch
    wg = synth.workload("grpo")
    cu = synth.cu_seqlens(synth.response_lengths(wg))
    T_tot = int(cu[-1])
    r = np.random.default_rng(4)
    lp_new = -np.abs(r.normal(0.5, 1.0, T_tot))
    lp_old = lp_new + r.normal(0, 0.05, T_tot)
    lp_ref = lp_new + r.normal(0, 0.1, T_tot)
    rw = synth.rewards(wg)
    t0 = time.perf_counter()
    OG.token_loss(lp_new, lp_old, lp_ref, cu, OG.advantages(rw, wg.group_size))
    dt = time.perf_counter() - t0
    _CPU_BASE["grpo_loss"] = {"value": T_tot / dt, "unit": "tokens/s", "cores": 1,
                              "kind": "oracle",
                              "sample": f"the GRPO/DAPO loss stage over all {T_tot} packed "
                                        f"tokens (advantages, ratios, clipped surrogate, k3, "
                                        f"gradient), fp64 numpy, one thread, {dt:.3f}s"}


def _host_bits(torch, t):
    """bf16 device tensor -> its uint16 bit patterns on the host."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def leg_logits(torch, rlk, synth, steps, warmup):
    w = synth.workload("qwen")
    t_gen = time.perf_counter()
    if "qwen" in _DATA:
        arr, y = _DATA["qwen"]
    else:
        arr = synth.logits_rows(w, range(w.N))
        y = synth.peak_targets(w, range(w.N))
    x = torch.from_numpy(arr.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    yt = torch.from_numpy(y).to("cuda:0")
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] logits leg: inputs {tuple(x.shape)} bf16 generated in {gen_s:.1f}s",
          file=sys.stderr, flush=True)
    fn = lambda: rlk.logprob_from_logits(x, yt, w.temperature, w.top_p)  # noqa: E731
    mean_ms, total_ms, min_ms, med_ms = _events_time(torch, fn, steps, warmup)
    det = _determinism(
        torch, fn, lambda idx: _outs(torch, rlk.logprob_from_logits(
            x[idx], yt[idx], w.temperature, w.top_p)), w.N, seed=2)
    rows = w.N
    bytes_per_row = 2 * w.V + 8 + 25     # logits + target id + 5 fp32, 1 int32, 1 flag out
    achieved = rows * bytes_per_row / (total_ms / steps * 1e-3) / 1e9
    res = {
        "workload": f"logits-in, {w.N} rows x V={w.V}, bf16 ~N(0,2.5^2)+1..32 peaks, "
                    f"T={w.temperature}, top-p={w.top_p}",
        "tokens_per_s": rows * steps / (total_ms * 1e-3),
        "ms_per_step": total_ms / steps,
        "per_call_ms_mean": mean_ms, "per_call_ms_median": med_ms, "per_call_ms_min": min_ms,
        "gpu_clock": _LAST_CLOCK[0],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _profile_traffic("bf16_hist_rows_qwen3_logits_4096x151936")},
        "bytes_per_row": bytes_per_row,
        "determinism": det,
    }
    if "logits" in _CPU_BASE:
        res["cpu_baseline"] = _CPU_BASE["logits"]
    return res


def leg_tiny(torch, rlk, synth, steps, warmup):
    """The small logits-in workload: 256 rows x 8192 fp32 logits ~N(0, 3^2),
    T=0.7, top-p=0.95 (8.4 MB: it stays in the 256 MB Infinity Cache, so the
    HBM roofline is reported, not a bound)."""
    w = synth.workload("tiny")
    if "tiny" in _DATA:
        arr, y = _DATA["tiny"]
    else:
        arr = synth.logits_rows(w, range(w.N))
        y = np.argmax(arr, axis=1).astype(np.int64)
    x = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to("cuda:0")
    yt = torch.from_numpy(y).to("cuda:0")
    fn = lambda: rlk.logprob_from_logits(x, yt, w.temperature, w.top_p)  # noqa: E731
    mean_ms, total_ms, min_ms, med_ms = _events_time(torch, fn, steps, warmup)
    det = _determinism(
        torch, fn, lambda idx: _outs(torch, rlk.logprob_from_logits(
            x[idx], yt[idx], w.temperature, w.top_p)), w.N, seed=1)
    bytes_per_row = 4 * w.V + 8 + 25
    achieved = w.N * bytes_per_row / (total_ms / steps * 1e-3) / 1e9
    res = {
        "workload": f"logits-in, {w.N} rows x V={w.V}, fp32 ~N(0,3^2), T={w.temperature}, "
                    f"top-p={w.top_p} (cache-resident: roofline reported, not graded)",
        "tokens_per_s": w.N * steps / (total_ms * 1e-3),
        "ms_per_step": total_ms / steps,
        "per_call_ms_mean": mean_ms, "per_call_ms_median": med_ms, "per_call_ms_min": min_ms,
        "gpu_clock": _LAST_CLOCK[0],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _profile_traffic("f32_rows_tiny_256x8192")},
        "bytes_per_row": bytes_per_row,
        "determinism": det,
    }
    if "tiny" in _CPU_BASE:
        res["cpu_oracle"] = _CPU_BASE["tiny"]
    return res


def leg_support(torch, rlk, synth, steps, warmup):
    """Retained-support scoring on the config-2 logits (4096 x 151936 bf16,
    T=0.7): each row's set is its top-p 0.95 nucleus (picked with torch
    outside the timed region: sort, tempered softmax, cumulative mass), as the
    rollout sampler would hand it over in CSR form; timed without and with the
    check against the recomputed nucleus."""
    w = synth.workload("qwen")
    arr = synth.logits_rows(w, range(w.N))
    y = synth.peak_targets(w, range(w.N))
    x = torch.from_numpy(arr.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    sets = []
    for r0 in range(0, w.N, 256):
        zs, idx = torch.sort(x[r0:r0 + 256].float() / w.temperature, dim=1, descending=True)
        c = torch.cumsum(torch.softmax(zs, dim=1), dim=1)
        k = (c < w.top_p).sum(dim=1) + 1
        for i in range(idx.shape[0]):
            sets.append(torch.sort(idx[i, :int(k[i])]).values.to(torch.int32))
    sizes = torch.tensor([t.numel() for t in sets], dtype=torch.int64)
    offsets = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(sizes, 0)]).to("cuda:0")
    ids = torch.cat(sets).contiguous()
    # targets: a member of each set (the first id), as a sampled token would be
    yt = torch.stack([t[0] for t in sets]).to(torch.int64).contiguous()
    nnz = int(ids.numel())
    del y
    print(f"[bench] support leg: {w.N} rows, {nnz} retained ids (median "
          f"{int(sizes.median())}, max {int(sizes.max())})", file=sys.stderr, flush=True)
    fn = lambda: rlk.logprob_from_support(x, yt, w.temperature, offsets, ids)  # noqa: E731
    mean_ms, total_ms, min_ms, med_ms = _events_time(torch, fn, steps, warmup)
    fnc = lambda: rlk.logprob_from_support(x, yt, w.temperature, offsets, ids,  # noqa: E731
                                           check_top_p=w.top_p)
    mean_c, total_c, min_c, med_c = _events_time(torch, fnc, max(3, steps // 4), warmup)
    det = _determinism(torch, fnc)
    from oracle import logprob as OL
    from oracle import support as OSup
    ns = w.N
    off_h = offsets[:ns + 1].cpu().numpy()
    ids_h, y_h = ids[:int(off_h[-1])].cpu().numpy(), yt[:ns].cpu().numpy()
    z_h = OL.widen_bf16(arr[:ns])
    cpu = _cpu_oracle(lambda: OSup.logprob_from_support(z_h, y_h, OL.f32(w.temperature), off_h,
                                                        ids_h), ns, f"all {ns} rows")
    # A gather moves whole 64-byte sectors: the bytes a perfect kernel must
    # move are the ids (4 B each), every distinct 64-byte sector of logits the
    # sets touch (32 bf16 ids per sector; a row's ids are sorted), and per row
    # the offsets, target and 9 B of outputs.
    sec = torch.div(ids, 32, rounding_mode="floor")
    same = sec[1:] == sec[:-1]
    starts = offsets[1:-1]
    same[starts[starts > 0] - 1] = False
    sectors = nnz - int(same.sum())
    alg = nnz * 4 + sectors * 64 + w.N * (8 + 8 + 9)
    achieved = alg / (total_ms / steps * 1e-3) / 1e9
    return {
        "workload": f"retained-support scoring, {w.N} rows x V={w.V} bf16, T={w.temperature}, "
                    f"sets = top-p {w.top_p} nuclei ({nnz} ids)",
        "tokens_per_s": w.N * steps / (total_ms * 1e-3),
        "ms_per_step": total_ms / steps,
        "per_call_ms_mean": mean_ms, "per_call_ms_median": med_ms, "per_call_ms_min": min_ms,
        "gpu_clock": _LAST_CLOCK[0],
        "distinct_64B_sectors": sectors,
        "with_nucleus_check_ms": total_c / max(3, steps // 4),
        "with_nucleus_check_tokens_per_s": w.N / (total_c / max(3, steps // 4) * 1e-3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 6),
                     "traffic": _profile_traffic("support_rows_qwen3_logits_4096x151936")},
        "determinism": det,
        "cpu_oracle": cpu,
    }


def leg_sample(torch, rlk, synth, steps, warmup):
    """Rollout-side top-p sampler on the config-2 logits (4096 x 151936 bf16,
    T=0.7, p=0.95): nucleus (row kernel), then the seeded Gumbel-max draw,
    which scores the drawn token with the row kernel's own statistics
    (bitwise the training-side value). Algorithmic bytes: one read of each
    row (2V) plus the outputs; the call reads each row twice (nucleus pass,
    then the draw), so the fraction counts the second read as overhead."""
    w = synth.workload("qwen")
    arr = synth.logits_rows(w, range(w.N))
    x = torch.from_numpy(arr.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    state = {"offset": 0}

    def fn():
        state["offset"] += 1
        return rlk.sample_top_p(x, w.temperature, w.top_p, 1234, state["offset"])

    mean_ms, total_ms, min_ms, med_ms = _events_time(torch, fn, steps, warmup)
    # with row keys = original row ids, a draw is a function of its row alone
    det = _determinism(
        torch, lambda: rlk.sample_top_p(x, w.temperature, w.top_p, 1234, 7),
        lambda idx: _outs(torch, rlk.sample_top_p(x[idx], w.temperature, w.top_p, 1234, 7,
                                                  row_keys=idx)), w.N, seed=3)
    from oracle import logprob as OL
    from oracle import sampling as OS
    ns = 64
    z_h = OL.widen_bf16(arr[:ns])
    Tf, pf = OL.f32(w.temperature), OL.f32(w.top_p)

    def oracle_draws():
        yd = np.array([OS.sample_row(z_h[n], Tf, pf, 1234, 7, n) for n in range(ns)])
        OL.logprob_from_logits(z_h, yd, Tf, pf)

    cpu = _cpu_oracle(oracle_draws, ns, f"first {ns} rows (draw and score)")
    bytes_per_row = 2 * w.V + 8 + 4 + 4 + 4 + 1
    achieved = w.N * bytes_per_row / (total_ms / steps * 1e-3) / 1e9
    return {
        "workload": f"top-p sampler + score, {w.N} rows x V={w.V} bf16, T={w.temperature}, "
                    f"top-p={w.top_p}, Philox-4x32-10 Gumbel-max",
        "tokens_per_s": w.N * steps / (total_ms * 1e-3),
        "ms_per_step": total_ms / steps,
        "per_call_ms_mean": mean_ms, "per_call_ms_median": med_ms, "per_call_ms_min": min_ms,
        "gpu_clock": _LAST_CLOCK[0],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _profile_traffic("sampler_qwen3_logits_4096x151936")},
        "bytes_per_row": bytes_per_row,
        "determinism": det,
        "cpu_oracle": cpu,
    }


def leg_fused(torch, rlk, synth, steps, warmup):
    """Fused LM-head forward, Qwen3-8B head: hidden [8192, 4096], W [151936, 4096], T=1, p=1."""
    w = synth.workload("fused")
    t_gen = time.perf_counter()
    hb = synth.hidden_rows(w, range(w.N))
    wb = synth.weight_rows(w, range(w.V))
    y = synth.uniform_targets(w, w.N)
    h = torch.from_numpy(hb.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    W = torch.from_numpy(wb.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    yt = torch.from_numpy(y).to("cuda:0")
    print(f"[bench] fused leg: hidden {tuple(h.shape)} W {tuple(W.shape)} generated in "
          f"{time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    fn = lambda: rlk.logprob_fused_linear(h, W, yt, w.temperature, 1.0)  # noqa: E731
    mean_ms, total_ms, min_ms, med_ms = _events_time(torch, fn, steps, warmup)
    det = _determinism(
        torch, fn, lambda idx: _outs(torch, rlk.logprob_fused_linear(
            h[idx], W, yt[idx], w.temperature, 1.0)), w.N, seed=3)
    from oracle import fused as OF
    from oracle import logprob as OL
    ns = 64
    W64 = OL.widen_bf16(wb)
    h64 = OL.widen_bf16(hb[:ns])
    cpu = _cpu_oracle(lambda: OF.forward(h64, W64, y[:ns], OL.f32(w.temperature), 1.0), ns,
                      f"first {ns} tokens", blas=True)
    del W64
    flops = 2.0 * w.N * w.V * w.H
    achieved = flops / (total_ms / steps * 1e-3) / 1e12
    return {
        "workload": f"fused LM-head forward, hidden [{w.N},{w.H}] bf16, W [{w.V},{w.H}] bf16, "
                    f"T={w.temperature}, top-p=1",
        "tokens_per_s": w.N * steps / (total_ms * 1e-3),
        "ms_per_step": total_ms / steps,
        "per_call_ms_mean": mean_ms, "per_call_ms_median": med_ms, "per_call_ms_min": min_ms,
        "gpu_clock": _LAST_CLOCK[0],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": _profile_traffic("fwd_tile_stats_qwen3_head_8192x4096x151936")},
        "flops_per_token": 2.0 * w.V * w.H,
        "determinism": det,
        "cpu_oracle": cpu,
    }


def leg_fused_bwd(torch, rlk, synth, steps, warmup):
    """Fused LM-head forward + backward, Llama-3-70B head: hidden [16384, 8192],
    W [128256, 8192], T=1, p=1, loss = -mean lp - 0.001 mean H (seeds
    g_lp = -1/N, g_H = -0.001/N)."""
    w = synth.workload("llama70b")
    t_gen = time.perf_counter()
    hb = synth.hidden_rows(w, range(w.N))
    wb = synth.weight_rows(w, range(w.V))
    y = synth.uniform_targets(w, w.N)
    h = torch.from_numpy(hb.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    W = torch.from_numpy(wb.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    del hb, wb
    yt = torch.from_numpy(y).to("cuda:0")
    g_lp = torch.full((w.N,), -1.0 / w.N, device="cuda:0")
    g_h = torch.full((w.N,), -0.001 / w.N, device="cuda:0")
    print(f"[bench] fused fwd+bwd leg: hidden {tuple(h.shape)} W {tuple(W.shape)} generated in "
          f"{time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)

    def step():
        out = rlk.logprob_fused_linear(h, W, yt, w.temperature, 1.0)
        return rlk.logprob_fused_linear_bwd(h, W, yt, out["saved"], g_lp, g_h, w.temperature, 1.0)

    mean_ms, total_ms, min_ms, med_ms = _events_time(torch, step, steps, warmup)

    def dh_rows(idx):   # dh of the rows idx (a row's dh depends on that row only; dW sums rows)
        hi, yi = h[idx], yt[idx]
        out = rlk.logprob_fused_linear(hi, W, yi, w.temperature, 1.0)
        return [rlk.logprob_fused_linear_bwd(hi, W, yi, out["saved"], g_lp[idx], g_h[idx],
                                             w.temperature, 1.0)[0]]

    det = _determinism(torch, step, dh_rows, w.N, seed=5)
    from oracle import fused as OF
    from oracle import logprob as OL
    ns = 8
    W64 = OL.widen_bf16(_host_bits(torch, W))
    h64 = OL.widen_bf16(_host_bits(torch, h[:ns]))
    gl, gh = np.full(ns, -1.0 / w.N), np.full(ns, -0.001 / w.N)

    def oracle_step():
        OF.forward(h64, W64, y[:ns], 1.0, 1.0)
        OF.backward(h64, W64, y[:ns], gl, gh, 1.0, 1.0)

    cpu = _cpu_oracle(oracle_step, ns, f"first {ns} tokens, forward and backward "
                                       "(dW: their contribution)", blas=True)
    del W64
    flops = 8.0 * w.N * w.V * w.H      # forward 2VH + recompute 2VH + dh 2VH + dW 2VH per token
    achieved = flops / (total_ms / steps * 1e-3) / 1e12
    return {
        "workload": f"fused LM-head forward+backward, hidden [{w.N},{w.H}] bf16, "
                    f"W [{w.V},{w.H}] bf16, T=1, top-p=1, loss -mean lp - 0.001 mean H",
        "tokens_per_s": w.N * steps / (total_ms * 1e-3),
        "ms_per_step": total_ms / steps,
        "per_call_ms_mean": mean_ms, "per_call_ms_median": med_ms, "per_call_ms_min": min_ms,
        "gpu_clock": _LAST_CLOCK[0],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": _profile_traffic("fused_fwd_bwd_llama70b_16384x8192x128256")},
        "flops_per_token_executed": 8.0 * w.V * w.H,
        "frac_useful_6vh": round(0.75 * achieved / BF16_PEAK_TFLOPS, 4),
        "determinism": det,
        "cpu_oracle": cpu,
    }


_GRPO_INPUTS = {}


def _grpo_inputs(torch, rlk, synth):
    """The config-4 batch (generated once per process): 32 packed responses
    (4 prompts x 8, lengths U{256..6912}), hidden/W, in-nucleus targets,
    old/ref logprobs (the new ones plus N(0, 0.05^2) / N(0, 0.1^2) noise),
    rewards."""
    if _GRPO_INPUTS:
        return _GRPO_INPUTS
    w = synth.workload("grpo")
    cu = synth.cu_seqlens(synth.response_lengths(w))
    T_tot = int(cu[-1])
    t_gen = time.perf_counter()
    hb = synth.hidden_rows(w, range(T_tot))
    wb = synth.weight_rows(w, range(w.V))
    h = torch.from_numpy(hb.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    W = torch.from_numpy(wb.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    del hb, wb
    # targets: each row's top token (always kept by the nucleus, so every
    # logprob and the loss are finite), from bf16 logits formed by torch
    # outside the timed region; the timing does not depend on which token
    yt = torch.empty(T_tot, dtype=torch.int64, device="cuda:0")
    for r0 in range(0, T_tot, 8192):
        yt[r0:r0 + 8192] = torch.mm(h[r0:r0 + 8192], W.t()).argmax(dim=1)
    print(f"[bench] grpo inputs: T_tot={T_tot} hidden {tuple(h.shape)} W {tuple(W.shape)} "
          f"generated in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    lp0 = rlk.logprob_fused_linear(h, W, yt, w.temperature, w.top_p)["logprob"]
    n_old, n_ref = synth.logprob_noise(w, T_tot)
    _GRPO_INPUTS.update(
        w=w, cu=cu, cu_dev=torch.from_numpy(cu).to("cuda:0"), T_tot=T_tot, h=h, W=W, yt=yt,
        lp_old=(lp0 + torch.from_numpy(n_old).to(lp0)).contiguous(),
        lp_ref=(lp0 + torch.from_numpy(n_ref).to(lp0)).contiguous(),
        rw=torch.from_numpy(synth.rewards(w)).to("cuda:0"))
    return _GRPO_INPUTS


def leg_grpo(torch, rlk, synth, steps, warmup):
    """Fused LM head at T=0.7, top-p=0.95 over the config-4 batch, H=4096,
    V=151936, then the GRPO/DAPO token loss."""
    g = _grpo_inputs(torch, rlk, synth)
    w, T_tot = g["w"], g["T_tot"]

    def step():
        out = rlk.logprob_fused_linear(g["h"], g["W"], g["yt"], w.temperature, w.top_p)
        return rlk.grpo_token_loss(out["logprob"], g["lp_old"], g["lp_ref"], g["cu_dev"],
                                   rewards=g["rw"], group_size=w.group_size)

    mean_ms, total_ms, min_ms, med_ms = _events_time(torch, step, steps, warmup)
    # the loss and its per-token outputs run to run; the top-p forward's
    # per-token outputs under splits and a permutation of the tokens
    det = _determinism(torch, step)
    det.update({k: v for k, v in _determinism(
        torch, lambda: rlk.logprob_fused_linear(g["h"], g["W"], g["yt"], w.temperature, w.top_p),
        lambda idx: _outs(torch, rlk.logprob_fused_linear(g["h"][idx], g["W"], g["yt"][idx],
                                                          w.temperature, w.top_p)),
        T_tot, seed=4).items() if k != "run_to_run_x3"})
    from oracle import fused as OF
    from oracle import grpo as OG
    from oracle import logprob as OL
    ns = 64
    W64 = OL.widen_bf16(_host_bits(torch, g["W"]))
    h64 = OL.widen_bf16(_host_bits(torch, g["h"][:ns]))
    y_h = g["yt"][:ns].cpu().numpy()
    lp_o, lp_r = g["lp_old"].cpu().numpy(), g["lp_ref"].cpu().numpy()
    r_h = g["rw"].cpu().numpy()
    Tf, pf = OL.f32(w.temperature), OL.f32(w.top_p)

    def oracle_grpo():   # forward on the sample; the loss stage over every token
        OF.forward(h64, W64, y_h, Tf, pf)
        OG.token_loss(lp_o, lp_o, lp_r, g["cu"], OG.advantages(r_h, w.group_size))

    cpu = _cpu_oracle(oracle_grpo, ns, f"first {ns} tokens of the top-p forward, plus the "
                                       f"loss stage over all {T_tot} tokens", blas=True)
    cpu_loss = _CPU_BASE.get("grpo_loss")
    del W64
    flops = 2.0 * T_tot * w.V * w.H
    achieved = flops / (total_ms / steps * 1e-3) / 1e12
    return {
        "workload": f"fused LM head top-p + GRPO loss, {T_tot} packed tokens (32 responses), "
                    f"H={w.H}, V={w.V}, T={w.temperature}, top-p={w.top_p}",
        "tokens_per_s": T_tot * steps / (total_ms * 1e-3),
        "ms_per_step": total_ms / steps,
        "per_call_ms_mean": mean_ms, "per_call_ms_median": med_ms, "per_call_ms_min": min_ms,
        "gpu_clock": _LAST_CLOCK[0],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": _profile_traffic("fused_topp_grpo_loss_109833_tokens")},
        "flops_per_token": 2.0 * w.V * w.H,
        "determinism": det,
        "cpu_oracle": cpu,
        "cpu_oracle_loss_stage": cpu_loss,
    }


def leg_grpo_train(torch, rlk, synth, steps, warmup):
    """A config-4 training step of the LM head: fused forward at top-p 0.95,
    the GRPO/DAPO token loss and its dL/dlogprob, then the fused backward
    through the same nucleus (dL/dhidden, dL/dW)."""
    g = _grpo_inputs(torch, rlk, synth)
    w, T_tot = g["w"], g["T_tot"]

    def step():
        out = rlk.logprob_fused_linear(g["h"], g["W"], g["yt"], w.temperature, w.top_p)
        loss = rlk.grpo_token_loss(out["logprob"], g["lp_old"], g["lp_ref"], g["cu_dev"],
                                   rewards=g["rw"], group_size=w.group_size)
        return rlk.logprob_fused_linear_bwd(g["h"], g["W"], g["yt"], out["saved"], loss["grad"],
                                            None, w.temperature, w.top_p)

    mean_ms, total_ms, min_ms, med_ms = _events_time(torch, step, steps, warmup)
    det = _determinism(torch, step)   # dh and dW, three steps bitwise
    from oracle import fused as OF
    from oracle import logprob as OL
    ns = 16
    W64 = OL.widen_bf16(_host_bits(torch, g["W"]))
    h64 = OL.widen_bf16(_host_bits(torch, g["h"][:ns]))
    y_h = g["yt"][:ns].cpu().numpy()
    Tf, pf = OL.f32(w.temperature), OL.f32(w.top_p)
    gl = np.full(ns, 1.0 / T_tot)

    def oracle_step():
        OF.forward(h64, W64, y_h, Tf, pf)
        OF.backward(h64, W64, y_h, gl, np.zeros(ns), Tf, pf)

    cpu = _cpu_oracle(oracle_step, ns, f"first {ns} tokens, top-p forward and backward "
                                       "(dW: their contribution)", blas=True)
    del W64
    flops = 8.0 * T_tot * w.V * w.H    # forward 2VH + recompute 2VH + dh 2VH + dW 2VH per token
    achieved = flops / (total_ms / steps * 1e-3) / 1e12
    return {
        "workload": f"LM-head GRPO training step: fused top-p forward + GRPO loss + backward "
                    f"through the nucleus, {T_tot} packed tokens, H={w.H}, V={w.V}, "
                    f"T={w.temperature}, top-p={w.top_p}",
        "tokens_per_s": T_tot * steps / (total_ms * 1e-3),
        "ms_per_step": total_ms / steps,
        "per_call_ms_mean": mean_ms, "per_call_ms_median": med_ms, "per_call_ms_min": min_ms,
        "gpu_clock": _LAST_CLOCK[0],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": _profile_traffic("grpo_train_step_109833_tokens")},
        "flops_per_token_executed": 8.0 * w.V * w.H,
        "determinism": det,
        "cpu_oracle": cpu,
    }


def leg_copy(torch, steps, warmup):
    """A plain 1 GiB device-to-device copy: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters (its algorithmic traffic is exactly
    1 GiB read + 1 GiB written per launch)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    mean_ms, total_ms, min_ms, med_ms = _events_time(torch, lambda: dst.copy_(src), steps, warmup)
    return {"workload": "device copy, 1 GiB", "bytes_read": n, "bytes_written": n,
            "per_call_ms_mean": mean_ms, "per_call_ms_median": med_ms, "per_call_ms_min": min_ms,
        "gpu_clock": _LAST_CLOCK[0],
            "tokens_per_s": 0.0, "ms_per_step": total_ms / steps,
            "roofline": {"bound": "hbm", "achieved": round(2 * n / (total_ms / steps * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(2 * n / (total_ms / steps * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": None}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--legs",
                    default="logits,tiny,support,sample,fused,grpo,grpo_train,fused_bwd")
    ap.add_argument("--cpu-sample", type=int, default=1,
                    help="0 = skip the CPU oracle timings (profiler runs)")
    ap.add_argument("--no-determinism", action="store_true",
                    help="skip the bitwise determinism checks (profiler runs)")
    args = ap.parse_args()
    _CHECK_DETERMINISM[0] = not args.no_determinism
    _CPU_ORACLE[0] = args.cpu_sample > 0
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1 "
                                   "(how the path would shard is described, not built)"}))
        sys.exit(2)

    import synth
    legs = [s for s in args.legs.split(",") if s]
    if args.cpu_sample > 0 and "logits" in legs:
        if _profiler_attached():
            print("[bench] CPU baselines skipped: a profiler is attached (it initialises "
                  "the GPU before this program starts, so no worker may be forked)",
                  file=sys.stderr, flush=True)
        else:
            cpu_baselines(synth)   # before the GPU is first used

    import torch
    import grpo_loss_rlk_amd as rlk

    out_legs = {}
    if "logits" in legs:   # the headline: a failure here fails the run
        out_legs["logits"] = leg_logits(torch, rlk, synth, args.steps, args.warmup)
    others = {
        "tiny": lambda: leg_tiny(torch, rlk, synth, args.steps, args.warmup),
        "support": lambda: leg_support(torch, rlk, synth, args.steps, args.warmup),
        "sample": lambda: leg_sample(torch, rlk, synth, max(3, args.steps // 4), args.warmup),
        "fused": lambda: leg_fused(torch, rlk, synth, min(20, max(3, args.steps // 4)), 1),
        "copy": lambda: leg_copy(torch, args.steps, args.warmup),
        "grpo": lambda: leg_grpo(torch, rlk, synth, 3, 1),
        "grpo_train": lambda: leg_grpo_train(torch, rlk, synth, 3, 1),
        "fused_bwd": lambda: leg_fused_bwd(torch, rlk, synth, 3, 1),
    }
    for name, run in others.items():
        if name not in legs:
            continue
        try:
            out_legs[name] = run()
        except Exception as e:  # noqa: BLE001 -- the other legs and the headline still report
            print(f"[bench] leg {name} failed: {type(e).__name__}: {e}", file=sys.stderr,
                  flush=True)
            out_legs[name] = {"error": f"{type(e).__name__}: {e}"}
        torch.cuda.empty_cache()
    ok_legs = [v for v in out_legs.values() if "error" not in v]
    if not ok_legs:
        print(json.dumps({"error": "no leg completed", "legs": out_legs}))
        sys.exit(1)
    main_leg = out_legs.get("logits") or ok_legs[0]
    line = {
        "metric": METRIC,
        "value": round(main_leg["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_leg["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and value distributions of the pages' Qwen3-8B workload)",
        "config": {"workload": main_leg["workload"]},
        "roofline": main_leg["roofline"],
        "cpu_baseline": main_leg.get("cpu_baseline"),
        # the metric's MFMA half: the fused LM-head forward at H = 4096, V = 151936
        "roofline_mfma": (out_legs.get("fused") or {}).get("roofline"),
        "tokens_per_s_fused": (out_legs.get("fused") or {}).get("tokens_per_s"),
        "legs": {k: {kk: vv for kk, vv in v.items() if kk != "cpu_baseline"}
                 for k, v in out_legs.items()},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
