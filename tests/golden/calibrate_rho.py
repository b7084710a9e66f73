"""Calibrate the token-correlation rho of the 35B decode-stack workload.

Test infrastructure: calls only the oracle and the seeded generators.

The stack's token inputs are an AR(1) sequence h0[t] = rho h0[t-1] +
sqrt(1 - rho^2) eps. The predicted layers (7..38) execute the set their
predecessor's head chose at the previous token, so how much consecutive
tokens share experts (what host staging must copy) depends on rho. This runs
the oracle free (its own routing and predictions, fp64) over the first tokens
for a list of rho values and prints the mean adjacent-token set overlap
|S_t & S_{t-1}| / K over the predicted layers.

    python tests/golden/calibrate_rho.py --tokens 32 --rho 0.5 0.9 0.99

The workload constants it fixes (the rho giving about 0.7 overlap and the one
giving about 0.25) are stored in sparse_moe_decode_amd/workloads.py.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
from sparse_moe_decode_amd import synth  # noqa: E402
from sparse_moe_decode_amd import workloads as wl  # noqa: E402


def overlap_run(los, roles, dm, toks, idx0, w0):
    """Free-running oracle over toks; returns [T, L, K] executed sets."""
    L, K = len(roles), dm["K"]
    pred_idx = {l: idx0[l] for l in range(L)}
    pred_w = {l: w0[l].astype(np.float64) for l in range(L)}
    prev = [None] * L
    sets = np.empty((len(toks), L, K), np.int32)
    for t in range(len(toks)):
        h16 = toks[t]
        new_pred = {}
        for l in range(L):
            out = los[l].step(h16, pred_idx[l], pred_w[l], prev[l])
            sets[t, l] = out["exec_idx"]
            prev[l] = out["exec_idx"].copy()
            if roles[l]["head"] and l + 1 < L:
                new_pred[l + 1] = (out["pred_idx"].copy(), out["pred_w"].copy())
            h16 = out["h_out"].astype(np.float16)
        for l, (pi, pw) in new_pred.items():
            pred_idx[l], pred_w[l] = pi, pw
    return sets


def mean_overlap(sets, layers, K):
    ov = [len(set(sets[t, l]) & set(sets[t - 1, l])) / K
          for t in range(1, sets.shape[0]) for l in layers]
    return float(np.mean(ov))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--tier", default="35b")
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=32)
    ap.add_argument("--rho", type=float, nargs="+", required=True)
    args = ap.parse_args()
    oracle.load()
    dm = synth.dims(args.tier)
    roles = synth.stack_roles(args.tier)
    L = len(roles)
    los = []
    for l, role in enumerate(roles):
        lw = synth.layer(args.seed, l, dm, role, zero_mean=True)
        los.append(oracle.LayerOracle(dm, lw))
        print(f"layer {l + 1}/{L} loaded", file=sys.stderr, flush=True)
    idx0, w0 = wl.initial_routing(args.tier, args.seed, L)
    cons = [l for l in range(L) if not roles[l]["router"]]
    results = {}

    def work(rho):
        t0 = time.perf_counter()
        toks = wl.token_inputs(args.tier, args.seed, args.tokens, rho)
        sets = overlap_run(los, roles, dm, toks, idx0, w0)
        results[rho] = dict(rho=rho, overlap_predicted=round(mean_overlap(sets, cons, dm["K"]), 4),
                            overlap_router=round(mean_overlap(
                                sets, [l for l in range(L) if l not in cons], dm["K"]), 4),
                            seconds=round(time.perf_counter() - t0, 1))
        print(json.dumps(results[rho]), flush=True)

    threads = [threading.Thread(target=work, args=(r,)) for r in args.rho]
    for th in threads:
        th.start()
    for th in threads:
        th.join()


if __name__ == "__main__":
    main()
