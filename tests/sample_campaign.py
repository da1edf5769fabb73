"""Large-count parity campaign of the draft-side draw (specv_sample): every
row of many seeded calls of one workload's draft rows, HIP library against the
fp64 oracle (oracle.sample_row), by the rules of tests/parity.py: tokens exact
unless the oracle's margin is below 1e-5 (and such mismatches fewer than 1e-4
of the rows); greedy rows and invalid temperatures exactly; row
log-normalisers to 1e-5 relative and argmaxes exactly.

Worker processes (spawned, CPU only) generate each call's rows from its seed
and run the oracle; the main process draws on the GPU and compares. It prints
one line per window of calls and writes a summary file.

    python tests/sample_campaign.py --workload b64_n5_v128256_bf16 --calls 320 --workers 16 --out FILE
"""

from __future__ import annotations

import argparse
import multiprocessing as mp
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

ROWS = 64


def _prepare(task):
    """Worker: one call's rows and the oracle's draw, argmax and log-normaliser for each."""
    import numpy as np

    import oracle
    import synth

    name, seed = task
    rows = synth.make_sample_rows(synth.workload(name), seed, ROWS)
    out = []
    for r in range(ROWS):
        z = synth.widen(rows.logits[r], rows.dtype)
        T = float(rows.temperature[r])
        res = oracle.sample_row(z, T, float(rows.uniforms[r]))
        L = oracle.tempered_log_normaliser(z[None, :], T)[0] if T > 0 else float("nan")
        out.append((res.token, res.margin, oracle.first_argmax(z), L))
    return seed, rows, out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--calls", type=int, required=True)
    ap.add_argument("--first-seed", type=int, default=1000)
    ap.add_argument("--workers", type=int, default=16)
    ap.add_argument("--out", required=True)
    args = ap.parse_args()

    import numpy as np
    import torch

    import parity
    import synth
    from speculative_sampling_verification_specv_amd import Verifier

    wl = synth.workload(args.workload)
    dev = parity.require_gpu()
    cases = exact = excused = 0
    hard = []
    t0 = time.time()
    seeds = list(range(args.first_seed, args.first_seed + args.calls))
    window = 2 * args.workers
    with Verifier(ROWS, 1, wl.vocab, wl.dtype) as v, \
            ProcessPoolExecutor(args.workers, mp_context=mp.get_context("spawn")) as ex:
        for w0 in range(0, len(seeds), window):
            for seed, rows, want in ex.map(_prepare, [(args.workload, s) for s in seeds[w0:w0 + window]]):
                a = np.ascontiguousarray(rows.logits)
                logits = (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if rows.dtype == "bf16"
                          else torch.from_numpy(a)).to(dev)
                toks = v.sample(logits, torch.from_numpy(rows.temperature).to(dev),
                                torch.from_numpy(rows.uniforms).to(dev))
                lse, amax = v.row_stats()
                torch.cuda.synchronize()
                toks, lse, amax = toks.cpu().numpy(), lse.cpu().numpy()[:, 0], amax.cpu().numpy()[:, 0]
                for r, (tok, margin, am, L) in enumerate(want):
                    cases += 1
                    T = float(rows.temperature[r])
                    info = dict(seed=seed, row=r, T=T, gpu=int(toks[r]), oracle=tok)
                    if parity.library_rejects_temperature(T):
                        ok = toks[r] == -1 and amax[r] == -1 and np.isnan(lse[r])
                    else:
                        ok = amax[r] == am and (np.isnan(lse[r]) if T == 0.0 else
                                                abs(float(lse[r]) - L) <= parity.LSE_RTOL * max(1.0, abs(L)))
                        if ok and toks[r] != tok:
                            if T > 0.0 and margin < parity.MARGIN:
                                excused += 1
                                continue
                            ok = False
                    if ok:
                        exact += 1
                    else:
                        hard.append(info)
            done = min(w0 + window, len(seeds))
            print(f"[sample campaign] {args.workload}: {done}/{len(seeds)} calls, rows={cases} exact={exact} "
                  f"excused={excused} hard={len(hard)} ({time.time() - t0:.0f} s)", flush=True)
    ok = not hard and excused <= parity.MAX_EXCUSED_RATE * cases
    lines = [
        f"# Sampling campaign (specv_sample): {args.workload} draft rows, {ROWS} rows per call, "
        f"seeds {seeds[0]}..{seeds[-1]} ({len(seeds)} calls), MI355X",
        f"# command: python tests/sample_campaign.py --workload {args.workload} --calls {args.calls} "
        f"--first-seed {args.first_seed} --workers {args.workers} --out <this file>",
        f"rows = {cases}",
        f"exact = {exact}",
        f"excused = {excused}  (fp64 margin < {parity.MARGIN})",
        f"hard = {len(hard)}",
        f"result = {'pass' if ok else 'FAIL'}",
    ]
    if hard:
        lines.append(f"first hard mismatches: {hard[:3]}")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
