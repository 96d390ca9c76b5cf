"""Worst errors seen by the GPU parity tests, per workload and stage, plus
per-layer drift curves; conftest.py writes them as JSON (parity_margins.json
in the run's output folder) when the session ends, so each run keeps its
margins against the bars."""
from __future__ import annotations

import json
import os

RECORD: dict = {}


def note(workload: str, stage: str, value: float, bar: float) -> None:
    """Keep the largest error seen for (workload, stage) and its bar."""
    ent = RECORD.setdefault(workload, {}).setdefault(stage, {"worst": 0.0, "bar": bar,
                                                            "checks": 0})
    ent["worst"] = max(ent["worst"], float(value))
    ent["bar"] = bar
    ent["checks"] += 1


def note_count(workload: str, key: str, n: int) -> None:
    ent = RECORD.setdefault(workload, {})
    ent[key] = int(ent.get(key, 0)) + int(n)


def note_series(workload: str, key: str, index, value) -> None:
    """Append one point (e.g. a layer's end-to-end walk drift) to a series."""
    RECORD.setdefault(workload, {}).setdefault(key, []).append([index, value])


def _short(x):
    """Three significant digits; series as {index: value} on one line each."""
    if isinstance(x, float):
        return float(f"{x:.3g}")
    if isinstance(x, dict):
        return {k: _short(v) for k, v in x.items()}
    if isinstance(x, list) and x and isinstance(x[0], list) and len(x[0]) == 2:
        return {(str(i) if not isinstance(i, list) else ",".join(map(str, i))): _short(v)
                for i, v in x}
    return x


def dump(path: str) -> None:
    if not RECORD:
        return
    os.makedirs(os.path.dirname(path), exist_ok=True)
    short = _short(RECORD)
    with open(path, "w") as f:
        f.write("{\n")
        items = sorted(short.items())
        for n, (wl, ent) in enumerate(items):
            f.write(f" {json.dumps(wl)}: {{\n")
            keys = sorted(ent)
            for m, k in enumerate(keys):
                sep = "," if m + 1 < len(keys) else ""
                f.write(f"  {json.dumps(k)}: {json.dumps(ent[k])}{sep}\n")
            f.write(" }" + ("," if n + 1 < len(items) else "") + "\n")
        f.write("}\n")
