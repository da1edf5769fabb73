#!/usr/bin/env python3
"""Throughput of batched speculative-sampling verification on one MI355X.

One step = one specv_verify call over one batch of the workload: row
statistics of every draft and target row, the accept scan and the residual or
bonus draw. Inputs are seeded synthetic logits already resident in HBM; several
copies of the logits are rotated so the 256 MB last-level cache cannot hold
the working set between steps.

Prints one JSON line: value = verified draft positions per second (B*N per
call), with the roofline of the dominant kernel (timed live with HIP events on
the launch stream) and the fp64 oracle timed on this host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "b64_n5_v128256_bf16"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
METRIC = "verified draft positions/sec and achieved HBM GB/s (% of peak), 1 MI355X"
KERNEL_SOURCE = os.path.join(ROOT, "speculative_sampling_verification_specv_amd", "csrc", "specv_kernels.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--copies", type=int, default=0, help="logit copies rotated per step (0: enough for 512 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of each oracle CPU baseline leg (single thread, then all cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also", default="b256_n7_v151936_bf16_mixed,b32_n16_v128256_f32",
                    help="comma-separated workloads also timed (reported under 'also'); empty for none")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the lines of the steps around the verification (lazy verification, draft-side "
                         "draw, acceptance rates, KV-cache commit)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MB (8 times) so that a "
                         "rocprofv3 --pmc run of this command also measures a copy of known size")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("PMC_DIR", "OUT"),
                    help="write the HBM traffic summary of the verification kernel from rocprofv3 --pmc "
                         "output (FETCH_SIZE and WRITE_SIZE runs under PMC_DIR) to OUT, then exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "OUT"),
                    help="write per-launch durations from a rocprofv3 --kernel-trace CSV, grouped by kernel "
                         "and grid size (the lazy and whole verifications share a kernel), to OUT, then exit")
    return ap.parse_args()


def algorithmic_bytes(batch, n_accepted) -> dict:
    """Bytes the method must read per call, split by kernel family.

    Row statistics read every row a sequence needs: 2N+1 rows at T > 0, the
    N+1 target rows at T = 0 (greedy never looks at draft rows). The draw
    re-reads target and draft row j after a rejection, target row N for the
    bonus, nothing when greedy.
    """
    B, N, V = batch.batch, batch.n_draft, batch.vocab
    e = 4 if batch.dtype == "f32" else 2
    T = batch.temperature
    sampled = (T > 0) & np.isfinite(T)
    greedy = T == 0
    stats_rows = int(sampled.sum()) * (2 * N + 1) + int(greedy.sum()) * (N + 1)
    resid = int((sampled & (n_accepted < N) & (n_accepted >= 0)).sum())
    bonus = int((sampled & (n_accepted == N)).sum())
    reread_rows = 2 * resid + bonus
    return dict(stats=stats_rows * V * e, reread=reread_rows * V * e,
                total=(stats_rows + reread_rows) * V * e, resid_seqs=resid, bonus_seqs=bonus,
                formula=B * (2 * N + 1) * V * e + reread_rows * V * e)


def _oracle_sequence(task):
    """Worker: the oracle, as it stands, on sequence s of the batch (inputs rebuilt from the seed)."""
    import oracle
    import synth

    name, seed, s = task
    batch = _cached_batch(name, seed)
    oracle.verify_sequence(synth.widen(batch.draft_logits[s], batch.dtype),
                           synth.widen(batch.target_logits[s], batch.dtype), batch.draft_tokens[s],
                           batch.accept_uniforms[s].astype(np.float64), float(batch.sample_uniforms[s]),
                           float(batch.temperature[s]))
    return 1


_BATCH_CACHE: dict = {}


def _cached_batch(name, seed):
    import synth

    key = (name, seed)
    if key not in _BATCH_CACHE:
        _BATCH_CACHE.clear()
        _BATCH_CACHE[key] = synth.make_batch(synth.workload(name), seed)
    return _BATCH_CACHE[key]


def _worker_init(name, seed):
    os.environ["OMP_NUM_THREADS"] = "1"
    _cached_batch(name, seed)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(batch, name: str, seed: int, budget_s: float) -> dict:
    """The fp64 oracle, as it stands, verifying whole sequences of this batch.

    Two legs of about ``budget_s`` each: one thread (sequences one after
    another in this process), then a process pool over sequences on every
    host core this process may use (capped at 16). The reported value is the
    all-core leg; the single-thread figure rides along.
    """
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import oracle
    import synth

    N = batch.n_draft
    done = 0
    t0 = time.perf_counter()
    while True:
        s = done % batch.batch
        oracle.verify_sequence(synth.widen(batch.draft_logits[s], batch.dtype),
                               synth.widen(batch.target_logits[s], batch.dtype), batch.draft_tokens[s],
                               batch.accept_uniforms[s].astype(np.float64), float(batch.sample_uniforms[s]),
                               float(batch.temperature[s]))
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    single = done * N / el
    cores = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1))
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(cores, mp_context=ctx, initializer=_worker_init, initargs=(name, seed)) as ex:
        # Warm the workers (each rebuilds the batch from its seed) outside the timed region.
        list(ex.map(_oracle_sequence, [(name, seed, s % batch.batch) for s in range(cores)]))
        n_par = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            chunk = [(name, seed, (n_par + k) % batch.batch) for k in range(4 * cores)]
            n_par += sum(ex.map(_oracle_sequence, chunk))
        el_par = time.perf_counter() - t0
    return {"value": n_par * N / el_par, "unit": "verified draft positions/sec", "cores": cores, "kind": "oracle",
            "cpu": cpu_model(), "single_thread_value": single,
            "sample": f"{n_par} sequences of this batch verified by the numpy fp64 oracle in {el_par:.1f} s on "
                      f"{cores} worker processes (one thread each); single thread: {done} sequences in {el:.1f} s"}


def traffic_record(kernel: str, workload: str):
    """HBM bytes per dispatch from committed rocprofv3 counter runs, if the kernel is unchanged since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256") != kernel_source_sha():
        return None
    return float(rec["hbm_bytes_per_dispatch"])


def kernel_source_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _pmc_rows(pmc_dir: str):
    """(dispatch id, kernel name, counter, value) of every dispatch in rocprofv3 counter CSVs under pmc_dir."""
    import csv

    for dirpath, _, files in os.walk(pmc_dir):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(dirpath, fn), newline="") as f:
                    for row in csv.DictReader(f):
                        yield (os.path.join(dirpath, fn), int(row["Dispatch_Id"])), row["Kernel_Name"], \
                            row["Counter_Name"], float(row["Counter_Value"])


def summarize_trace(trace_csv: str, out: str) -> int:
    """Launch durations of this library's kernels in a rocprofv3 kernel trace,
    one line per (kernel, grid size): count, mean, median, min and max in us."""
    import csv

    groups: dict = {}
    with open(trace_csv, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            if not re.search(r"\b(verify|sample|rate_parts|rate_finish|kv_commit)_kernel\b|narrow_to_float|zero_words",
                             name):
                continue
            short = name
            if short.endswith(")"):  # drop the parameter list: back to the parenthesis matching the last one
                depth = 0
                for i in range(len(short) - 1, -1, -1):
                    depth += {")": 1, "(": -1}.get(short[i], 0)
                    if depth == 0:
                        short = short[:i]
                        break
            short = short.split("::")[-1]
            key = (short, int(row["Grid_Size_X"]))
            groups.setdefault(key, []).append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    lines = ["# kernel, grid size (work-items), launches, mean / median / min / max duration (us)\n"]
    for (short, grid), d in sorted(groups.items()):
        a = np.asarray(d)
        lines.append(f"{short}, {grid}, {a.size}, {a.mean():.2f} / {np.median(a):.2f} / {a.min():.2f} / "
                     f"{a.max():.2f}\n")
    with open(out, "w") as f:
        f.writelines(lines)
    return 0


def summarize_pmc(pmc_dir: str, out: str, workload: str, copy_mb: int, kernel: str = "verify") -> int:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of one kernel, scaled by a plain copy's.

    The calibration copies are the first 8 __amd_rocclr_copyBuffer dispatches of
    each run (bench.py --calibrate-copy-mb makes them before anything else is
    copied); each moves copy_mb * 10^6 bytes each way. The ratio of that to what
    the same counter reads for them is the factor applied to the verify kernel.
    """
    verify: dict = {}
    copies: dict = {}
    for key, name, ctr, val in sorted(_pmc_rows(pmc_dir)):
        if f"{kernel}_kernel" in name:
            verify.setdefault(ctr, []).append(val)
        elif "copyBuffer" in name:
            seen = copies.setdefault((key[0], ctr), [])
            if len(seen) < 8:
                seen.append(val)
    copy_vals: dict = {}
    for (_, ctr), vals in copies.items():
        copy_vals.setdefault(ctr, []).extend(vals)
    need = ["FETCH_SIZE", "WRITE_SIZE"]
    missing = [c for c in need if c not in verify or len(copy_vals.get(c, [])) < 8]
    if missing:
        print(f"counters missing in {pmc_dir}: {missing}", file=sys.stderr)
        return 1
    mean = {("verify", c): float(np.mean(verify[c])) for c in need}
    mean.update({("copy", c): float(np.mean(copy_vals[c])) for c in need})
    copy_bytes = copy_mb * 1e6
    f_fetch = copy_bytes / (mean[("copy", "FETCH_SIZE")] * 1024.0)
    f_write = copy_bytes / (mean[("copy", "WRITE_SIZE")] * 1024.0)
    fetch = mean[("verify", "FETCH_SIZE")] * 1024.0 * f_fetch
    write = mean[("verify", "WRITE_SIZE")] * 1024.0 * f_write
    text = "".join([
        f"# HBM traffic of {kernel}_kernel, workload {workload}, from two rocprofv3 --pmc runs\n",
        "# (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, mean over the dispatches of the run),\n",
        f"# each scaled by the factor that maps the same counter on a plain {copy_mb} MB device copy\n",
        "# (__amd_rocclr_copyBuffer, the run's first 8 copies) to its known size.\n",
        f"kernel_dispatches = {len(verify['FETCH_SIZE'])}\n",
        f"kernel_fetch_kib_per_dispatch = {mean[('verify', 'FETCH_SIZE')]:.1f}\n",
        f"kernel_write_kib_per_dispatch = {mean[('verify', 'WRITE_SIZE')]:.1f}\n",
        f"copy_fetch_kib_per_dispatch = {mean[('copy', 'FETCH_SIZE')]:.1f}\n",
        f"copy_write_kib_per_dispatch = {mean[('copy', 'WRITE_SIZE')]:.1f}\n",
        f"copy_bytes_per_dispatch = {copy_bytes:.0f}\n",
        f"fetch_scale = {f_fetch:.4f}\n",
        f"write_scale = {f_write:.4f}\n",
        f"hbm_fetch_bytes_per_dispatch = {fetch:.0f}\n",
        f"hbm_write_bytes_per_dispatch = {write:.0f}\n",
        f"hbm_bytes_per_dispatch = {fetch + write:.0f}\n",
        f"kernel_source_sha256 = {kernel_source_sha()}\n",
    ])
    with open(out, "w") as f:
        f.write(text)
    print(text, end="")
    return 0


def calibration_copy(torch, dev, mb: int) -> None:
    """A plain device-to-device copy of mb * 10^6 bytes, 8 times (the counters' scale reference)."""
    n = mb * 1000 * 1000
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def device_logits(torch, a, dtype, dev):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(a)
    return t.to(dev)


def lazy_bytes(batch, n_accepted) -> dict:
    """Rows the lazy verification reads: for each sequence the draft and target
    rows of every stage up to the one where it ends (stages [0,2), [2,8),
    [8,32), ..., or [0,2), [2,4), [4,8), ... when one position of the batch
    is 96 MB or more), target row N if that is the last stage, plus the draw's
    re-read (as for the full path)."""
    B, N, V = batch.batch, batch.n_draft, batch.vocab
    e = 4 if batch.dtype == "f32" else 2
    growth = 2 if B * V * e * 2 >= 96_000_000 else 4
    stages, lo = [], 0
    while lo < N:
        hi = min(N, 2) if lo == 0 else min(N, growth * lo)
        stages.append((lo, hi))
        lo = hi
    rows = 0
    for s in range(B):
        T, j = float(batch.temperature[s]), int(n_accepted[s])
        if j < 0 or not np.isfinite(T) or T < 0:
            continue
        hi_last = [hi for lo, hi in stages if lo <= min(j, N - 1)][-1]
        rows += hi_last * (2 if T > 0 else 1) + (1 if hi_last == N else 0)
    reread = algorithmic_bytes(batch, n_accepted)["reread"]
    return dict(stats=rows * V * e, reread=reread, total=rows * V * e + reread)


def measure(torch, dev, name: str, args, lazy: bool = False) -> dict:
    """Time K calls of workload `name`; returns the numbers the JSON line reports."""
    import synth
    from speculative_sampling_verification_specv_amd import Verifier

    wl = synth.WORKLOADS[name]
    batch = synth.make_batch(wl, args.seed)
    B, N, V = batch.batch, batch.n_draft, batch.vocab
    copy_bytes = B * (2 * N + 1) * V * wl.elem_bytes
    copies = args.copies or max(3, math.ceil(512e6 / copy_bytes))
    d0 = device_logits(torch, batch.draft_logits, batch.dtype, dev)
    t0_ = device_logits(torch, batch.target_logits, batch.dtype, dev)
    sets = [(d0, t0_)] + [(d0.clone(), t0_.clone()) for _ in range(copies - 1)]
    small = dict(draft_tokens=torch.from_numpy(batch.draft_tokens).to(dev),
                 accept_uniforms=torch.from_numpy(batch.accept_uniforms).to(dev),
                 sample_uniforms=torch.from_numpy(batch.sample_uniforms).to(dev),
                 temperature=torch.from_numpy(batch.temperature).to(dev))
    out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((B,), dtype=torch.int32, device=dev)
    v = Verifier(B, N, V, batch.dtype)

    # Each input copy's call is checked once and then re-enqueued directly
    # (what a serving loop that refills its buffers does), so the timed loop
    # measures the GPU, not Python's per-call argument checks.
    calls = [v.bind(d, t, out_tokens=out_tokens, out_n_accepted=out_n, lazy=lazy, **small) for d, t in sets]

    def step(k):
        calls[k % copies]()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    n_acc = out_n.cpu().numpy()
    nbytes = algorithmic_bytes(batch, n_acc)
    if lazy:
        nbytes = dict(nbytes, **lazy_bytes(batch, n_acc))

    # Timed region: K whole calls, bracketed by device synchronisation, with
    # HIP events on the launch stream (torch's current stream, which the
    # binding passes) around the same K launches: the kernel's average
    # duration is their elapsed time / K, on the same basis as ms_per_step.
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(args.steps):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    kernel_ms = e0.elapsed_time(e1) / args.steps
    v.close()
    # Algorithmic bytes of the launch: every row the method needs once, plus
    # the draw's re-read of the drawn row(s) (the finishers' load of one
    # member's tokens per sequence is counted with them).
    kernel_bytes = nbytes["stats"] + nbytes["reread"]
    dominant = "verify"
    stage_ms = {dominant: kernel_ms}
    return dict(
        workload=name, batch=batch, copies=copies, ms_per_step=ms_per_step, nbytes=nbytes,
        stage_ms=stage_ms, dominant=dominant, kernel_bytes=kernel_bytes,
        achieved=kernel_bytes / (stage_ms[dominant] * 1e-3) / 1e9,
        positions=B * N, n_accepted_mean=float(np.mean(n_acc)),
    )


def _time_calls(torch, dev, step, steps: int, warmup: int) -> float:
    """Mean ms of one call over `steps` back-to-back calls (events on the launch stream)."""
    for k in range(warmup):
        step(k)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(steps):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _direct(fn, *args):
    """A call of a C entry point with its arguments marshalled once (the
    binding's checks would otherwise bound the timed loop by Python's speed)."""
    from speculative_sampling_verification_specv_amd import _lib

    def call(_k=0):
        rc = fn(*args)
        if rc != _lib.SPECV_OK:
            raise _lib.SpecvError(rc, fn.__name__)
    return call


def measure_extras(torch, dev, args) -> dict:
    """The steps around the verification, each on a workload-shaped input:
    lazy verification (the long-draft and 64-sequence workloads), the
    draft-side draw (the 64-sequence workload's draft rows), acceptance rates
    after a verification, and the KV-cache commit of the accepted drafts."""
    import synth
    from speculative_sampling_verification_specv_amd import Verifier, _lib

    out = {}
    for name in ("b32_n16_v128256_f32", "b64_n5_v128256_bf16"):
        m = measure(torch, dev, name, args, lazy=True)
        out[f"lazy_{name}"] = {
            "positions_per_sec": m["positions"] / (m["ms_per_step"] * 1e-3), "ms_per_step": m["ms_per_step"],
            "bytes_per_call": m["nbytes"]["total"], "hbm_gbs": m["nbytes"]["total"] / (m["ms_per_step"] * 1e-3) / 1e9,
            "mean_n_accepted": m["n_accepted_mean"]}
    # Draft-side draw: 64 rows of the 64-sequence bf16 workload's draft logits.
    wl = synth.workload("b64_n5_v128256_bf16")
    rows = synth.make_sample_rows(wl, args.seed, 64)
    V = wl.vocab
    row_bytes = 64 * V * 2
    copies = max(3, math.ceil(512e6 / row_bytes))
    base = torch.from_numpy(np.ascontiguousarray(rows.logits).view(np.int16)).view(torch.bfloat16).to(dev)
    logit_sets = [base] + [base.clone() for _ in range(copies - 1)]
    temp = torch.from_numpy(rows.temperature).to(dev)
    uni = torch.from_numpy(rows.uniforms).to(dev)
    tok = torch.empty(64, dtype=torch.int32, device=dev)
    with Verifier(64, 1, V, "bf16") as v:
        v.sample(logit_sets[0], temp, uni, tok)  # the binding's checks, once
        lib = _lib.load_library()
        calls = [_direct(lib.specv_sample, v.handle, 64, _lib._ptr(x), _lib._ptr(temp), _lib._ptr(uni), _lib._ptr(tok),
                         _lib._stream_ptr(None, dev)) for x in logit_sets]
        ms = _time_calls(torch, dev, lambda k: calls[k % copies](), args.steps, args.warmup)
    # One pass over each row (plus the finisher's load of one member's 4096 tokens per row).
    out["sample_b64_v128256_bf16"] = {"rows_per_sec": 64 / (ms * 1e-3), "ms_per_call": ms,
                                      "bytes_per_call": row_bytes,
                                      "hbm_gbs": row_bytes / (ms * 1e-3) / 1e9}
    del logit_sets
    # Acceptance rates after a verification (64-sequence workload). The rates
    # read the rows again; copies of the same logits are rotated (the
    # verification's row statistics hold for each), so the rows come from HBM.
    batch = synth.make_batch(wl, args.seed)
    d = device_logits(torch, batch.draft_logits, batch.dtype, dev)
    t = device_logits(torch, batch.target_logits, batch.dtype, dev)
    n_copies = max(3, math.ceil(512e6 / (d.numel() * 2 + t.numel() * 2)))
    sets = [(d, t)] + [(d.clone(), t.clone()) for _ in range(n_copies - 1)]
    small = dict(draft_tokens=torch.from_numpy(batch.draft_tokens).to(dev),
                 accept_uniforms=torch.from_numpy(batch.accept_uniforms).to(dev),
                 sample_uniforms=torch.from_numpy(batch.sample_uniforms).to(dev),
                 temperature=torch.from_numpy(batch.temperature).to(dev))
    B, N = batch.batch, batch.n_draft
    with Verifier(B, N, V, batch.dtype) as v:
        _, n_acc = v.verify(d, t, **small)
        alpha, tau = v.acceptance_rates(d, t, small["draft_tokens"], small["temperature"])  # checks, once
        lib = _lib.load_library()
        calls = [_direct(lib.specv_acceptance_rates, v.handle, B, N, _lib._ptr(dd), _lib._ptr(tt),
                         _lib._ptr(small["draft_tokens"]), _lib._ptr(small["temperature"]), _lib._ptr(alpha),
                         _lib._ptr(tau), _lib._stream_ptr(None, dev)) for dd, tt in sets]
        ms = _time_calls(torch, dev, lambda k: calls[k % n_copies](), args.steps, args.warmup)
        n_acc = n_acc.cpu().numpy()
    del sets
    rate_bytes = B * 2 * N * V * 2
    out["rates_b64_n5_v128256_bf16"] = {"ms_per_call": ms, "bytes_per_call": rate_bytes,
                                        "hbm_gbs": rate_bytes / (ms * 1e-3) / 1e9}
    # KV-cache commit of the accepted drafts of that batch: 32 layers of keys and
    # values (64 planes) of 8 heads x 128 bf16 (2 KB per entry), cache of 256.
    P, E, L = 64, 2048, 256
    cache = torch.empty((P, B, L, E // 2), dtype=torch.bfloat16, device=dev)
    scratch = torch.randn((P, B, N, E // 2), device=dev).to(torch.bfloat16)
    n_t = torch.from_numpy(n_acc.astype(np.int32)).to(dev)
    lens = torch.full((B,), 100, dtype=torch.int32, device=dev)
    new_len = torch.empty_like(lens)
    _lib.specv_kv_commit(cache, lens, scratch, n_t, new_len)  # the binding's checks, once
    es = cache.element_size()
    kv = _direct(_lib.load_library().specv_kv_commit, P, B, N, L, E, _lib._ptr(cache), cache.stride(0) * es,
                 cache.stride(1) * es, _lib._ptr(scratch), scratch.stride(0) * es, scratch.stride(1) * es,
                 _lib._ptr(n_t), _lib._ptr(lens), _lib._ptr(new_len), _lib._stream_ptr(None, dev))
    ms = _time_calls(torch, dev, lambda k: kv(), args.steps, args.warmup)
    kv_bytes = 2 * int(np.clip(n_acc, 0, None).sum()) * P * E
    out["kv_commit_b64_p64_e2048"] = {"ms_per_call": ms, "bytes_per_call": kv_bytes,
                                      "hbm_gbs": kv_bytes / (ms * 1e-3) / 1e9,
                                      "entries_committed": int(np.clip(n_acc, 0, None).sum()) * P}
    return out


def main() -> int:
    args = parse()
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                             args.calibrate_copy_mb or 256)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace[0], args.summarize_trace[1])
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sequences shard across GPUs with no exchange but the outputs); run with --gpus 1",
              file=sys.stderr)
        return 2

    import torch

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda", 0)
    if args.calibrate_copy_mb:
        calibration_copy(torch, dev, args.calibrate_copy_mb)

    m = measure(torch, dev, args.workload, args)
    batch, nbytes = m["batch"], m["nbytes"]
    B, N, V = batch.batch, batch.n_draft, batch.vocab
    ms = m["ms_per_step"]
    line = {
        "metric": METRIC,
        "value": m["positions"] / (ms * 1e-3),
        "unit": "verified draft positions/sec",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": batch.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "n_draft": N, "vocab": V, "logits": batch.dtype,
                   "temperature": sorted(set(float(x) for x in batch.temperature)), "seed": args.seed,
                   "rotated_copies": m["copies"]},
        "path": {
            "hbm_gbs": nbytes["total"] / (ms * 1e-3) / 1e9,
            "hbm_frac": nbytes["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_call": nbytes["total"],
            "formula_bytes_per_call": nbytes["formula"],
            "residual_seqs": nbytes["resid_seqs"],
            "bonus_seqs": nbytes["bonus_seqs"],
            "mean_n_accepted": m["n_accepted_mean"],
            "kernel_ms": m["stage_ms"][m["dominant"]],
            "kernel_bytes_per_launch": m["kernel_bytes"],
        },
        "roofline": {"bound": "hbm", "kernel": m["dominant"], "achieved": m["achieved"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": m["achieved"] / HBM_PEAK_GBS,
                     "traffic": traffic_record(m["dominant"], args.workload)},
    }
    also = {}
    for name in [x for x in args.also.split(",") if x and x != args.workload]:
        a = measure(torch, dev, name, args)
        also[name] = {
            "positions_per_sec": a["positions"] / (a["ms_per_step"] * 1e-3),
            "ms_per_step": a["ms_per_step"],
            "bytes_per_call": a["nbytes"]["total"],
            "formula_bytes_per_call": a["nbytes"]["formula"],
            "hbm_gbs": a["nbytes"]["total"] / (a["ms_per_step"] * 1e-3) / 1e9,
            "kernel_ms": a["stage_ms"][a["dominant"]],
            "kernel_achieved_gbs": a["achieved"],
            "kernel_frac": a["achieved"] / HBM_PEAK_GBS,
            "traffic": traffic_record(a["dominant"], name),
        }
    if also:
        line["also"] = also
    if not args.no_extras:
        line["extras"] = measure_extras(torch, dev, args)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(batch, args.workload, args.seed, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
