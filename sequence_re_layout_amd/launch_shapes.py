"""Measured launch shapes of the named workloads, kept in a table.

``launch_shapes.json`` (beside this module) maps a workload name and a mode
("basp" or "ulysses") to the tuning of each direction (the fields of
``basp_tuning``), as ``bench.py --tune-shapes`` measured them on an MI355X:
``basp_plan_autotune`` run several times per plan, and the resulting pairs
of shapes (with the built-in one) timed as whole back-to-back steps replayed
from HIP graphs, the fastest kept.  Reading the shapes from the table lets
the benchmark, its kernel traces, its counter runs and the parity tests run
the same kernel instances, instead of each autotuning anew.

Only launch shapes are stored: the re-layout's result does not depend on
them, only its speed does.
"""
from __future__ import annotations

import json
import os

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "launch_shapes.json")


def table(path: str = PATH) -> dict:
    """The whole table ({} when the file does not exist)."""
    try:
        with open(path) as f:
            return json.load(f)
    except FileNotFoundError:
        return {}


def lookup(name: str, mode: str, path: str = PATH):
    """(seq_to_head, head_to_seq) tuning dicts of a workload and mode, or
    None when the table has no entry for it."""
    entry = table(path).get("shapes", {}).get(name, {}).get(mode)
    if not entry:
        return None
    return entry["seq_to_head"], entry["head_to_seq"]


def apply(b, plan, name: str, mode: str, path: str = PATH) -> bool:
    """Set a plan's two directions to the table's shapes; False (plan
    unchanged) when the table has no entry.  ``b`` is the binding module."""
    found = lookup(name, mode, path)
    if found is None:
        return False
    b.basp_plan_set_direction_tuning(plan, b.BASP_SEQ_TO_HEAD, **found[0])
    b.basp_plan_set_direction_tuning(plan, b.BASP_HEAD_TO_SEQ, **found[1])
    return True
