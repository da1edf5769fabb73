"""Large-count parity campaign: every sequence of many seeded calls of one
workload, HIP library against the fp64 oracle, by the rules of tests/parity.py.

The GPU tests check a few hundred cases per workload; resolving the excused
mismatch bound (fewer than 1e-4 of cases, each with an fp64 margin below
1e-5) takes about 2e4 cases per workload, which this script runs outside
pytest. Worker processes (spawned, CPU only) generate each call's inputs from
its seed and run the oracle on all of its sequences; the main process runs
the library on the same inputs and compares. With --lazy every call also runs
specv_verify_lazy on the same device inputs, and its tokens and counts are
compared with the oracle by the same rules. It prints one line per window of
calls and writes a summary file.

    python tests/parity_campaign.py --workload b64_n5_v128256_bf16 --calls 313 --workers 16 --out FILE
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


def _prepare(task):
    """Worker: one call's inputs and the oracle's result for every sequence."""
    import numpy as np

    import oracle
    import synth

    name, seed = task
    b = synth.make_batch(synth.workload(name), seed)
    res = [oracle.verify_sequence(synth.widen(b.draft_logits[s], b.dtype), synth.widen(b.target_logits[s], b.dtype),
                                  b.draft_tokens[s], b.accept_uniforms[s].astype(np.float64),
                                  float(b.sample_uniforms[s]), float(b.temperature[s]))
           for s in range(b.batch)]
    return seed, b, res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--calls", type=int, required=True)
    ap.add_argument("--first-seed", type=int, default=1000)
    ap.add_argument("--workers", type=int, default=16)
    ap.add_argument("--out", required=True)
    ap.add_argument("--lazy", action="store_true", help="also compare the lazy verification")
    args = ap.parse_args()

    import parity
    import synth
    from speculative_sampling_verification_specv_amd import Verifier

    import torch

    wl = synth.workload(args.workload)
    device = parity.require_gpu()
    total = parity.Tally()
    lazy_total = parity.Tally()
    t0 = time.time()
    seeds = list(range(args.first_seed, args.first_seed + args.calls))
    window = 2 * args.workers  # calls in flight: bounds the inputs held in memory
    with Verifier(wl.batch, wl.n_draft, wl.vocab, wl.dtype) as ver, \
            ProcessPoolExecutor(args.workers, mp_context=mp.get_context("spawn")) as ex:
        for w0 in range(0, len(seeds), window):
            for seed, b, res in ex.map(_prepare, [(args.workload, s) for s in seeds[w0:w0 + window]]):
                gpu = parity.run_gpu(b, ver, device)
                t = parity.compare(b, gpu, res)
                total = total.merge(t)
                if args.lazy:
                    toks, nacc = ver.verify_lazy(**parity.to_device(b, device))
                    torch.cuda.synchronize()
                    lz = parity.GpuResult(toks.cpu().numpy(), nacc.cpu().numpy(), None, None)
                    lazy_total = lazy_total.merge(parity.compare(b, lz, res))
            done = min(w0 + window, len(seeds))
            extra = (f"; lazy exact={lazy_total.exact} excused={lazy_total.excused} hard={len(lazy_total.hard)}"
                     if args.lazy else "")
            print(f"[campaign] {args.workload}: {done}/{len(seeds)} calls, cases={total.cases} "
                  f"exact={total.exact} excused={total.excused} hard={len(total.hard)}{extra} "
                  f"({time.time() - t0:.0f} s)", flush=True)
    bound = parity.MAX_EXCUSED_RATE
    ok = not total.hard and total.excused <= bound * total.cases
    if args.lazy:
        ok = ok and not lazy_total.hard and lazy_total.excused <= bound * lazy_total.cases
    lines = [
        f"# Parity campaign: {args.workload}, seeds {seeds[0]}..{seeds[-1]} ({len(seeds)} calls), MI355X",
        f"# command: python tests/parity_campaign.py --workload {args.workload} --calls {args.calls} "
        f"--first-seed {args.first_seed} --workers {args.workers}{' --lazy' if args.lazy else ''} --out <this file>",
        f"cases = {total.cases}",
        f"exact = {total.exact}",
        f"excused = {total.excused}  (fp64 margin < {parity.MARGIN} at the first divergence)",
        f"hard = {len(total.hard)}",
        f"excused_rate = {total.excused / max(1, total.cases):.2e}  (bound {parity.MAX_EXCUSED_RATE:.0e})",
    ]
    if args.lazy:
        lines += [
            f"lazy_cases = {lazy_total.cases}",
            f"lazy_exact = {lazy_total.exact}",
            f"lazy_excused = {lazy_total.excused}",
            f"lazy_hard = {len(lazy_total.hard)}",
        ]
    lines.append(f"result = {'pass' if ok else 'FAIL'}")
    if total.hard:
        lines.append(f"first hard mismatches: {total.hard[:3]}")
    if args.lazy and lazy_total.hard:
        lines.append(f"first lazy hard mismatches: {lazy_total.hard[:3]}")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
