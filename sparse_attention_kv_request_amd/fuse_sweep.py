"""The measurements behind the copy inside the plan kernel: step times of
three builds of the same sources on the same box, alternated.

* ``separate``: ``-DHISPARSE_FUSE_MIN_ROWS=1000000000`` -- every call uses the
  separate miss-copy kernel;
* ``fused_u8``: ``-DHISPARSE_FUSE_MIN_ROWS=1`` -- every token-row call copies
  inside the plan kernel, 8 loads in flight per lane (the default unroll);
* ``fused_u4``: the same with ``-DHISPARSE_FUSE_UNROLL=4``.

(Page mode always uses the separate kernel; its rows measure the cost of the
plan kernel's unused copy branch, i.e. nothing.)

``python -m sparse_attention_kv_request_amd.fuse_sweep build`` (CPU) writes
the three libraries under ``_build/fuse_sweep/``; ``python -m
sparse_attention_kv_request_amd.fuse_sweep run`` (GPU) times, for each build in
turn (two rounds), the eager step of the headline workload at 8, 16, 32 and
64 requests (8 layers) and of workloads 1, 3, 4 and 5, and prints a markdown
table of the per-case medians.
"""
from __future__ import annotations

import json
import pathlib
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]
OUT = ROOT / "_build" / "fuse_sweep"
VARIANTS = {
    "separate": ["-DHISPARSE_FUSE_MIN_ROWS=1000000000"],
    "fused_u8": ["-DHISPARSE_FUSE_MIN_ROWS=1"],
    "fused_u4": ["-DHISPARSE_FUSE_MIN_ROWS=1", "-DHISPARSE_FUSE_UNROLL=4"],
}
CASES = [(2, 8), (2, 16), (2, 32), (2, 64), (3, None), (4, None), (5, None), (1, None)]


def build():
    from sparse_attention_kv_request_amd import build as b

    for name, defines in VARIANTS.items():
        b.build(verbose=True, defines=defines, lib=OUT / name / "libhisparse.so")


def _measure(lib_path):
    """One process per build: eager step times (ms) of every case."""
    sys.path.insert(0, str(ROOT))
    import torch

    import bench
    from sparse_attention_kv_request_amd import binding, workloads

    binding.LIB_PATH = pathlib.Path(lib_path)
    torch.cuda.set_device(0)
    res = {}
    for cfg, B in CASES:
        W, K = (5, 10) if cfg != 1 else (3, 12)
        over = {"steps": W + K}
        if B is not None:
            over["batch"] = B
        w = workloads.config(cfg, **over)
        run = bench.Runner(torch, binding, workloads, w)
        el, _, _ = run.timed(W, K, profile=False)
        run.close()
        res[f"{cfg}/{B or w.batch}"] = el * 1e3 / K
    print(json.dumps(res), flush=True)


def run(rounds=2):
    import statistics

    for name in VARIANTS:
        if not (OUT / name / "libhisparse.so").exists():
            raise SystemExit(f"{OUT / name} is missing: run this module's build step first")
    got = {name: [] for name in VARIANTS}
    for r in range(rounds):
        for name in VARIANTS:
            p = subprocess.run([sys.executable, "-m", "sparse_attention_kv_request_amd.fuse_sweep",
                                "measure", str(OUT / name / "libhisparse.so")],
                               cwd=ROOT, capture_output=True, text=True, timeout=900)
            if p.returncode:
                raise SystemExit(p.stderr[-2000:])
            got[name].append(json.loads(p.stdout.strip().splitlines()[-1]))
            print(f"round {r} {name} done", file=sys.stderr, flush=True)
    keys = list(got["separate"][0])
    names = {"2": "headline workload", "1": "workload 1", "3": "workload 3 (CLOCK, 4 steps)",
             "4": "workload 4", "5": "workload 5 (pages)"}
    print("| case (workload / requests) | " + " | ".join(f"{n} ms/step" for n in VARIANTS) +
          " | fused_u8 vs separate |")
    print("|---" * (len(VARIANTS) + 2) + "|")
    for k in keys:
        med = {n: statistics.median(x[k] for x in got[n]) for n in VARIANTS}
        cfg, B = k.split("/")
        print(f"| {names[cfg]}, {B} requests | " +
              " | ".join(f"{med[n]:.4f}" for n in VARIANTS) +
              f" | {100 * (med['fused_u8'] / med['separate'] - 1):+.1f} % |")


def main():
    if len(sys.argv) >= 2 and sys.argv[1] == "build":
        build()
    elif len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) >= 3 and sys.argv[1] == "measure":
        _measure(sys.argv[2])
    else:
        raise SystemExit("usage: python -m sparse_attention_kv_request_amd.fuse_sweep "
                         "build|run")


if __name__ == "__main__":
    main()
