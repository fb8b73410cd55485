"""X-ray analysis of one decode step's per-workgroup, per-phase records.

The monolith page (milestone M2) turns a dump of per-block phase stamps into
per-phase time, wait time per block, idle time per SM and bandwidth per
phase, after aligning the per-SM clocks.  Here every record carries
s_memrealtime stamps (a 100 MHz counter common to all XCDs, used for the
timeline) and s_memtime stamps (the shader clock, used for the finer
within-phase split between waiting and working).

`budget()` splits the step into the page's budget-bar categories: weight
GEMVs (QKV, O, gate/up, down), waits for inputs, attention (+ merge), and the
LM head + argmax.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

RT_NS = 10.0   # s_memrealtime tick in ns (100 MHz)
KINDS = ("qkv", "attention", "merge", "o_proj", "gate_up", "down")


def phase_name(phase: int, n_layers: int) -> str:
    if phase == 1:
        return "embed"
    if phase == 6 * n_layers + 2:
        return "lm_head"
    if phase == 6 * n_layers + 3:
        return "argmax"
    return KINDS[(phase - 2) % 6]


def memtime_per_ns(rec: np.ndarray) -> float:
    """Shader-clock ticks per ns, from the records' own paired stamps."""
    dt = (rec["t_end"].astype(np.float64) - rec["t_start"])
    drt = (rec["rt_end"].astype(np.float64) - rec["rt_start"]) * RT_NS
    ok = drt > 2000
    return float(np.median(dt[ok] / drt[ok])) if ok.any() else 2.4


def phase_table(rec: np.ndarray, n_layers: int) -> Dict[int, dict]:
    """Per phase id: wall span across workgroups (realtime), and over the
    active workgroups the median duration and median wait (shader clock)."""
    rec = rec[rec["rt_start"] > 0]
    f = memtime_per_ns(rec)
    t0 = rec["rt_start"].min()
    out = {}
    for ph in np.unique(rec["phase"]):
        r = rec[rec["phase"] == ph]
        act = r[r["active"] == 1]
        use = act if len(act) else r
        dur = (use["t_end"].astype(np.float64) - use["t_start"]) / f
        wait = (use["t_wait_end"].astype(np.float64) - use["t_wait_begin"]) / f
        pre = (use["t_wait_begin"].astype(np.float64) - use["t_start"]) / f
        marks = {}
        for k in range(4):
            mk = use["t_mark"][:, k].astype(np.float64)
            okm = mk > 0
            if okm.any():
                marks[f"mark{k}_after_wait_ns"] = float(np.median((mk[okm] - use["t_wait_end"][okm]) / f))
        out[int(ph)] = {
            "name": phase_name(int(ph), n_layers),
            "start_ns": float((r["rt_start"].min() - t0) * RT_NS),
            "end_ns": float((r["rt_end"].max() - t0) * RT_NS),
            "span_ns": float((r["rt_end"].max() - r["rt_start"].min()) * RT_NS),
            "active_wgs": int(len(act)),
            "median_dur_ns": float(np.median(dur)),
            "median_wait_ns": float(np.median(wait)),
            "median_before_wait_ns": float(np.median(pre)),
            "max_wait_ns": float(np.max(wait)),
            **marks,
        }
    return out


def budget(rec: np.ndarray, n_layers: int) -> dict:
    """Split one step into weight GEMV work, input waits, attention and the
    LM head, using the median active workgroup of each phase.  Phases run
    back to back per workgroup, so the category totals add up to about the
    step's length."""
    tab = phase_table(rec, n_layers)
    cats = {"weight_gemv_ns": 0.0, "wait_ns": 0.0, "attention_ns": 0.0, "lm_head_ns": 0.0, "other_ns": 0.0}
    per_kind: Dict[str, float] = {}
    for ph, t in tab.items():
        name, dur, wait = t["name"], t["median_dur_ns"], t["median_wait_ns"]
        per_kind[name] = per_kind.get(name, 0.0) + dur
        if name in ("qkv", "o_proj", "gate_up", "down"):
            cats["wait_ns"] += wait
            cats["weight_gemv_ns"] += max(dur - wait, 0.0)
        elif name in ("attention", "merge"):
            cats["attention_ns"] += dur
        elif name in ("lm_head", "argmax"):
            cats["wait_ns"] += wait
            cats["lm_head_ns"] += max(dur - wait, 0.0)
        else:
            cats["other_ns"] += dur
    rr = rec[rec["rt_start"] > 0]
    step_ns = float((rr["rt_end"].max() - rr["rt_start"].min()) * RT_NS)
    out = {"step_ns": step_ns, **{k: round(v, 1) for k, v in cats.items()},
           "per_phase_kind_ns": {k: round(v, 1) for k, v in per_kind.items()}}
    return out
