"""Summarise a rocprofv3 kernel-trace database as a short markdown table.

``python -m sparse_attention_kv_request_amd.profile_summary RESULTS.db
--skip N --command "..."`` prints, per kernel, the launch count and the
average duration over all launches and over the launches after the first
``N`` of that kernel (the warm-up launches a benchmark does not time), so the
figure matches what the benchmark measures live.
"""
from __future__ import annotations

import argparse
import collections
import re
import sqlite3


def short(name: str) -> str:
    m = re.search(r"::(\w+)(<[^()]*>)?\(", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return name.split("(")[0][:60]


def summarize(db_path: str, skip: int, limit: int = 0, skip_for=None):
    """Per kernel: (name, launches, mean us, timed launches, timed mean us,
    total us); the timed launches are those after the first `skip` (or
    skip_for[name]) of that kernel, at most `limit` of them."""
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, duration from kernels order by start").fetchall()
    by = collections.OrderedDict()
    for name, dur in rows:
        by.setdefault(short(name), []).append(dur / 1e3)  # ns -> us
    out = []
    for k, v in by.items():
        sk = next((n for pre, n in (skip_for or {}).items() if k.startswith(pre)), skip)
        timed = v[sk:] if len(v) > sk else v
        if limit:
            timed = timed[:limit]
        out.append((k, len(v), sum(v) / len(v), len(timed), sum(timed) / len(timed), sum(v)))
    out.sort(key=lambda r: -r[5])
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--skip", type=int, default=0)
    ap.add_argument("--limit", type=int, default=0,
                    help="use at most this many launches per kernel after the skipped ones")
    ap.add_argument("--skip-for", action="append", default=[], metavar="KERNEL=N",
                    help="another skip count for kernels whose short name starts with KERNEL")
    ap.add_argument("--command", default="")
    ap.add_argument("--title", default="rocprofv3 kernel trace")
    a = ap.parse_args()
    print(f"# {a.title}\n")
    if a.command:
        print(f"Command: `{a.command}`\n")
    skip_for = dict((s.split("=")[0], int(s.split("=")[1])) for s in a.skip_for)
    if skip_for:
        print("Skipped launches per kernel: " + ", ".join(f"`{k}` {n}" for k, n in skip_for.items())
              + f", others {a.skip}; at most {a.limit or 'all'} timed launches each.\n")
    print(f"| kernel | launches | avg us (all) | launches timed | avg us (timed) | total us |")
    print("|---|---|---|---|---|---|")
    for k, n, avg, nt, avg_t, tot in summarize(a.db, a.skip, a.limit, skip_for):
        print(f"| `{k}` | {n} | {avg:.2f} | {nt} | {avg_t:.2f} | {tot:.1f} |")


if __name__ == "__main__":
    main()
