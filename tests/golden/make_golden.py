"""Writes the oracle's final sampled motion for selected clips of the full-size
workloads to tests/golden/sample_c{config}_clip{b}.npz.

Calls only oracle/ and synthetic/ (never the HIP library). Clips are
independent from noise to x_0 (each clip's CFG pair runs its own chain), so a
clip of a batched workload is computed by running the oracle at B = 1 on that
clip's text, noise and length. Each file stores x_0 [T, 279] (float32) with the
metadata the GPU tests check before comparing arrays: config, clip, length,
seeds, steps, guidance scale, model depth and dtype, and the SHA-256 of the
oracle source it was made with.

    python tests/golden/make_golden.py [--jobs 4] [--only c1,c2]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

# two BLAS threads per worker process, set before numpy is first imported (the
# workers are forked from this process and keep its thread pool size)
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS"):
    os.environ.setdefault(_var, "2")

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

# (config, clip selection rule)
TARGETS = {
    "c1": (1, "all"),
    "c2": (2, "all"),
    "c3": (3, "spread8"),
    "c4": (4, "padded4_full4"),
}


def clips_for(config: int, rule: str):
    import numpy as np

    from synthetic.inputs import CONFIGS, make_lengths

    c = CONFIGS[config]
    lens = make_lengths(c["B"], c["T"], c["lengths"])
    if rule == "all":
        return list(range(c["B"]))
    if rule == "spread8":
        # the shortest and longest clip, the first and last of the batch (the
        # ends of the packed rows), and the clips at the length quartiles
        order = [int(i) for i in np.argsort(lens, kind="stable")]
        picks = [order[0], order[-1], 0, c["B"] - 1] + [order[(len(order) * q) // 4] for q in (1, 2, 3)]
        picks = list(dict.fromkeys(picks))
        picks += [i for i in (order[(len(order) * q) // 8] for q in (1, 3, 5, 7)) if i not in picks][:8 - len(picks)]
        return sorted(picks)
    if rule == "padded4_full4":
        # four padded clips (the first, the last, the shortest and one in the
        # middle of the padded set) and four full-length ones (first, last and
        # two in the middle of the batch)
        padded = [int(i) for i in (lens < c["T"]).nonzero()[0]]
        full = [int(i) for i in (lens == c["T"]).nonzero()[0]]
        shortest = min(padded, key=lambda i: (lens[i], i))
        picks = [padded[0], padded[-1], shortest] + [i for i in padded[len(padded) // 2:] if i != shortest][:1]
        picks = list(dict.fromkeys(picks))
        picks += [i for i in padded if i not in picks][:4 - len(picks)]
        fpick = [full[0], full[-1], full[len(full) // 3], full[(2 * len(full)) // 3]]
        return sorted(dict.fromkeys(picks + fpick))
    raise ValueError(rule)


def oracle_sha() -> str:
    with open(os.path.join(ROOT, "oracle", "kimodo_oracle.py"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def golden_path(config: int, clip: int) -> str:
    return os.path.join(HERE, f"sample_c{config}_clip{clip}.npz")


def run_one(config: int, clip: int) -> str:
    import numpy as np

    from oracle import kimodo_oracle as O
    from synthetic.inputs import config_inputs

    ci = config_inputs(config)
    t0 = time.time()
    x0 = O.run_config_sample(ci["weights"], ci["dims"], ci["noise"][clip:clip + 1], ci["text"][clip:clip + 1],
                             ci["lengths"][clip:clip + 1], ci["steps"], ci["cfg_scale"])
    meta = dict(config=config, clip=clip, length=int(ci["lengths"][clip]), B=ci["B"], T=ci["T"],
                steps=ci["steps"], cfg_scale=ci["cfg_scale"], layers=ci["layers"], dtype=ci["dtype"],
                seeds=dict(weights=0, text=1, noise=2, lengths=3), oracle_sha256=oracle_sha(),
                seconds=round(time.time() - t0, 1))
    path = golden_path(config, clip)
    np.savez_compressed(path, x0=x0[0].astype(np.float32), meta=json.dumps(meta))
    return f"{path} ({meta['seconds']} s)"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--only", default=",".join(TARGETS))
    args = ap.parse_args()
    work = []
    for key in args.only.split(","):
        config, rule = TARGETS[key]
        work += [(config, clip) for clip in clips_for(config, rule)]
    with ProcessPoolExecutor(max_workers=args.jobs) as ex:
        for msg in ex.map(run_one, *zip(*work)):
            print(msg, flush=True)


if __name__ == "__main__":
    main()
