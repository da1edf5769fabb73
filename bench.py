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
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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


def cpu_baseline(batch, budget_s: float) -> dict:
    """The fp64 oracle, as it stands, on whole sequences of this batch until the budget is spent."""
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
    return {"value": done * N / el, "unit": "verified draft positions/sec", "cores": 1, "kind": "oracle",
            "sample": f"{done} sequences of this batch verified one after another by the numpy fp64 oracle "
                      f"(single thread) in {el:.1f} s"}


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
    with open(KERNEL_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    return float(rec["hbm_bytes_per_dispatch"])


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sequences shard across GPUs with no exchange but the outputs); run with --gpus 1",
              file=sys.stderr)
        return 2

    import torch

    import synth
    from speculative_sampling_verification_specv_amd import Verifier

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda", 0)
    wl = synth.WORKLOADS[args.workload]
    batch = synth.make_batch(wl, args.seed)
    B, N, V = batch.batch, batch.n_draft, batch.vocab
    e = wl.elem_bytes
    copy_bytes = B * (2 * N + 1) * V * e
    copies = args.copies or max(3, math.ceil(512e6 / copy_bytes))

    def logits(a):
        a = np.ascontiguousarray(a)
        if batch.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
        return torch.from_numpy(a)

    d_host, t_host = logits(batch.draft_logits), logits(batch.target_logits)
    sets = [(d_host.to(dev), t_host.to(dev)) for _ in range(copies)]
    small = dict(draft_tokens=torch.from_numpy(batch.draft_tokens).to(dev),
                 accept_uniforms=torch.from_numpy(batch.accept_uniforms).to(dev),
                 sample_uniforms=torch.from_numpy(batch.sample_uniforms).to(dev),
                 temperature=torch.from_numpy(batch.temperature).to(dev))
    out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((B,), dtype=torch.int32, device=dev)
    v = Verifier(B, N, V, batch.dtype)

    def step(k):
        d, t = sets[k % copies]
        v.verify(d, t, out_tokens=out_tokens, out_n_accepted=out_n, **small)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    n_acc = out_n.cpu().numpy()
    nbytes = algorithmic_bytes(batch, n_acc)

    # Timed region: K whole calls, bracketed by device synchronisation.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        step(k)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    ms_events = start.elapsed_time(end) / args.steps

    # Per-kernel durations: HIP events the library records around each kernel
    # on the launch stream (a separate pass; recording adds a little overhead).
    v.set_timing(True)
    sums = {}
    for k in range(args.steps):
        step(k)
        for name, ms in v.last_timings().items():
            sums[name] = sums.get(name, 0.0) + ms
    v.set_timing(False)
    stage_ms = {k: s / args.steps for k, s in sums.items()}
    dominant = max(stage_ms, key=stage_ms.get)
    kernel_bytes = {"row_stats": nbytes["stats"]}.get(dominant, nbytes["reread"])
    achieved = kernel_bytes / (stage_ms[dominant] * 1e-3) / 1e9
    traffic = traffic_record(dominant, args.workload)

    positions = B * N
    line = {
        "metric": METRIC,
        "value": positions / (ms_per_step * 1e-3),
        "unit": "verified draft positions/sec",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": batch.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "n_draft": N, "vocab": V, "logits": batch.dtype,
                   "temperature": sorted(set(float(x) for x in batch.temperature)), "seed": args.seed,
                   "rotated_copies": copies},
        "path": {
            "hbm_gbs": nbytes["total"] / (ms_per_step * 1e-3) / 1e9,
            "hbm_frac": nbytes["total"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_call": nbytes["total"],
            "formula_bytes_per_call": nbytes["formula"],
            "ms_per_step_events": ms_events,
            "residual_seqs": nbytes["resid_seqs"],
            "bonus_seqs": nbytes["bonus_seqs"],
            "stage_ms": stage_ms,
        },
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    v.close()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
