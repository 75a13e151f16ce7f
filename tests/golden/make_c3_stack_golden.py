"""Write the stored oracle values for the 50-block denoising step at full size.

Calls only ``oracle`` (the CPU reference) and ``seeded_inputs`` (the seeded
draws both sides use); nothing here comes from the GPU path.

Workload: 50 stacked AdaLN DiT blocks of 22680 tokens (the 864x480, 56-frame
latent: 14 frames of 30 x 54), hidden 5120, 40 heads x 128, MLP 13824,
bf16-rounded inputs, every block with its own seeded weights ~ N(0, 0.02^2),
zero biases, one shared c, x ~ N(0, 1).  A denoising step runs 50 blocks, or
the first 45 under the reduced layer count (h3.c memory-techniques page,
technique 2; h3-metal review, knob list).

The stack is run in segments through ``oracle.stack_forward`` with the blocks
generated one at a time as the stack asks for them (all 50 blocks at once
would need 80 GB of fp32 weights).  Running blocks a..b-1 on the state after
block a is the same computation as the full stack, block by block.  The state
after blocks 1, 10, 25, 45 and 50 is stored at a fixed sample of token rows
(the first 8, the last 8, which include the ragged tail of 22680 = 88 * 256 +
152, and 16 drawn with seed 5).

Usage: python tests/golden/make_c3_stack_golden.py [--state-dir DIR]
With --state-dir, the full fp32 state after each segment is kept there and a
rerun resumes from the last one.  About 1.5 h on 8 host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import seeded_inputs as si  # noqa: E402

OUT_NPZ = os.path.join(HERE, "c3_stack_n22680_d5120_rows.npz")
OUT_JSON = os.path.join(HERE, "c3_stack_n22680_d5120_rows.json")
CHECKPOINTS = (1, 10, 25, 45, 50)
N_SAMPLE = 32
ROW_SEED = 5


def sample_rows(n: int) -> np.ndarray:
    rng = np.random.default_rng(ROW_SEED)
    head = list(range(8))
    tail = list(range(n - 8, n))
    mid = rng.choice(np.arange(8, n - 8), size=N_SAMPLE - 16, replace=False).tolist()
    return np.array(sorted(set(head + tail + mid)), dtype=np.int64)


class LazyBlocks:
    """Blocks first .. first+count-1 of the step, drawn when the stack asks."""

    def __init__(self, shape, first: int, count: int):
        self.shape, self.first, self.count = shape, first, count

    def __len__(self):
        return self.count

    def __getitem__(self, i):
        if not 0 <= i < self.count:
            raise IndexError(i)
        l = self.first + i
        t = time.perf_counter()
        w = {k: v.values for k, v in si.gen_block_weights(self.shape, l).items()}
        print(f"  block {l}: weights drawn in {time.perf_counter() - t:.1f} s", flush=True)
        return w


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--state-dir", default=None)
    args = ap.parse_args()

    shape = si.C3
    hx, hc = si.gen_activation(shape)
    x = hx.values
    c = hc.values
    rows = sample_rows(shape.n_tokens)
    states = {}
    done = 0
    if args.state_dir:
        os.makedirs(args.state_dir, exist_ok=True)
        for l in reversed(CHECKPOINTS):
            p = os.path.join(args.state_dir, f"state_{l}.npy")
            if os.path.exists(p):
                x = np.load(p)
                done = l
                break
        for l in CHECKPOINTS:
            if l <= done:
                states[l] = np.load(os.path.join(args.state_dir, f"state_{l}.npy"))[rows]
    t_all = time.perf_counter()
    timings = {}
    for l in CHECKPOINTS:
        if l <= done:
            continue
        t = time.perf_counter()
        x = oracle.stack_forward(x, c, LazyBlocks(shape, done, l - done), shape.n_heads)
        dt = time.perf_counter() - t
        timings[f"blocks_{done}_{l}_s"] = round(dt, 1)
        print(f"blocks {done}..{l - 1}: {dt:.1f} s, state rms {float(np.sqrt(np.mean(x.astype(np.float64) ** 2))):.3f}",
              flush=True)
        states[l] = x[rows].copy()
        if args.state_dir:
            np.save(os.path.join(args.state_dir, f"state_{l}.npy"), x)
        done = l

    np.savez(OUT_NPZ, rows=rows, **{f"state_after_{l}": states[l] for l in CHECKPOINTS})
    meta = {
        "what": "fp32 oracle state of the 50-block AdaLN DiT stack (22680 tokens, hidden 5120, 40 heads x 128, "
                "MLP 13824) after blocks 1, 10, 25, 45 and 50, at the token rows in 'rows'.",
        "inputs": "seeded_inputs workload c3: config id 3, base seed 42, x and c ~ N(0,1), weights ~ N(0, 0.02^2) "
                  "per block (SeedSequence([42, 3, block, tensor])), zero biases, all rounded to bf16 (RNE).",
        "writer": "tests/golden/make_c3_stack_golden.py (oracle.stack_forward in segments)",
        "checkpoints": list(CHECKPOINTS),
        "rows": rows.tolist(),
        "host": {"machine": platform.machine(), "processor": platform.processor(), "cores": len(os.sched_getaffinity(0)),
                 "numpy": np.__version__},
        "timings_s": timings,
        "total_s": round(time.perf_counter() - t_all, 1),
    }
    with open(OUT_JSON, "w") as f:
        json.dump(meta, f, indent=1)
    print("wrote", OUT_NPZ, OUT_JSON, flush=True)


if __name__ == "__main__":
    main()
