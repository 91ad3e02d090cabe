"""Worst measured error of every GPU parity check, kept for the end-of-session summary.

Each check calls ``record(label, quantity, error, bound)``; ``tests/conftest.py`` prints
the table after the run (also under ``pytest -q``), and writes it as JSON lines to the
file named by the ``KPAGE_PARITY_RECORD`` environment variable when that is set.
"""
from __future__ import annotations

import json
import os
from typing import List, Tuple

RECORDS: List[Tuple[str, str, float, float, str]] = []


def record(label: str, quantity: str, error: float, bound: float, note: str = "") -> None:
    RECORDS.append((label, quantity, float(error), float(bound), note))


def summary_lines() -> List[str]:
    if not RECORDS:
        return []
    w = max(len(r[0]) for r in RECORDS)
    out = [f"{'check':<{w}}  quantity  worst error  bound      error/bound  note"]
    for label, qty, err, bound, note in RECORDS:
        ratio = err / bound if bound > 0 else float("inf")
        out.append(f"{label:<{w}}  {qty:<8}  {err:11.3e}  {bound:9.3e}  {ratio:11.3f}  {note}")
    return out


def dump() -> None:
    path = os.environ.get("KPAGE_PARITY_RECORD")
    if not path or not RECORDS:
        return
    with open(path, "a") as f:
        for label, qty, err, bound, note in RECORDS:
            f.write(json.dumps({"check": label, "quantity": qty, "error": err, "bound": bound, "note": note}) + "\n")
