"""X-ray analysis of one decode step's per-workgroup, per-phase records.

The monolith page (milestone M2) turns a dump of per-block phase stamps into
per-phase time, wait time per block and idle time, after aligning the clocks.
Here every stamp is s_memrealtime (100 MHz, one counter for all XCDs), so no
alignment is needed.  Per workgroup and phase the kernel records when its
courier began gathering the phase's input (t_start), when every word of it
was present (t_ready), when it was handed to the compute waves (t_handoff),
when the first compute wave saw it (t_seen) and when the last one had
published its outputs (t_done).

The step is a chain: embed -> per layer QKV -> attention -> O -> gate/up ->
down -> LM head -> argmax.  For each phase of the chain:

* t_in      the last producer of its input published (the previous phase's
            latest t_done);
* exchange  t_in -> t_ready, median over consumers: the words' trip through
            the memory system plus the courier's polling;
* handoff   t_ready -> t_seen (courier transform, LDS hand-off);
* compute   t_seen -> t_done (dot products on weights already in registers,
            any wait for weights still in flight, and the stores);
* phase     t_in -> the phase's latest t_done: its share of the step.

`budget()` sums these over the chain into the page's budget-bar categories:
weight GEMVs, waits for inputs (exchange + hand-off), attention, and the LM
head + argmax.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

RT_NS = 10.0   # s_memrealtime tick in ns (100 MHz)
KINDS = ("qkv", "attention", "merge", "o_proj", "gate_up", "down")
LAYER_CHAIN = (0, 1, 3, 4, 5)   # phase offsets in a layer, in dependency order


def phase_name(phase: int, n_layers: int) -> str:
    if phase == 1:
        return "embed"
    if phase == 6 * n_layers + 2:
        return "lm_head"
    if phase == 6 * n_layers + 3:
        return "argmax"
    return KINDS[(phase - 2) % 6]


def chain(n_layers: int) -> List[int]:
    out = [1]
    for l in range(n_layers):
        out += [2 + 6 * l + k for k in LAYER_CHAIN]
    return out + [6 * n_layers + 2, 6 * n_layers + 3]


def _ns(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64) * RT_NS


def phase_table(rec: np.ndarray, n_layers: int) -> Dict[int, dict]:
    """Per phase of the chain: the exchange / hand-off / compute split (ns,
    medians over the workgroups that had work) and its span on the step's
    critical path."""
    rec = rec[rec["active"] == 1]
    if len(rec) == 0:
        return {}
    t0 = float(rec["t_start"][rec["t_start"] > 0].min()) * RT_NS
    out: Dict[int, dict] = {}
    t_in = t0
    for ph in chain(n_layers):
        r = rec[rec["phase"] == ph]
        if len(r) == 0:
            continue
        ready = _ns(r["t_ready"])
        hand = _ns(r["t_handoff"])
        seen = _ns(r["t_seen"])
        done = _ns(r["t_done"])
        has_ready = ready > 0
        has_seen = seen > 0
        has_done = done > 0
        end = float(done[has_done].max()) if has_done.any() else float(hand.max())
        row = {
            "name": phase_name(ph, n_layers),
            "active_wgs": int(len(r)),
            "t_in_ns": t_in - t0,
            "end_ns": end - t0,
            "phase_ns": end - t_in,
        }
        if has_ready.any():
            row["exchange_ns"] = float(np.median(ready[has_ready])) - t_in
            row["exchange_max_ns"] = float(ready[has_ready].max()) - t_in
        ok = has_ready & has_seen
        if ok.any():
            row["handoff_ns"] = float(np.median(seen[ok] - ready[ok]))
        ok = has_seen & has_done
        if ok.any():
            row["compute_ns"] = float(np.median(done[ok] - seen[ok]))
            row["compute_max_ns"] = float((done[ok] - seen[ok]).max())
        out[int(ph)] = row
        t_in = end
    return out


def budget(rec: np.ndarray, n_layers: int) -> dict:
    """Split the step's critical path into weight-GEMV work, waits for inputs
    (exchange + hand-off), attention, and LM head + argmax.  The categories
    add up to the step's length from the first stamp to the argmax."""
    tab = phase_table(rec, n_layers)
    cats = {"weight_gemv_ns": 0.0, "wait_ns": 0.0, "attention_ns": 0.0, "lm_head_ns": 0.0, "other_ns": 0.0}
    per_kind: Dict[str, float] = {}
    for ph, t in tab.items():
        name, span = t["name"], t["phase_ns"]
        per_kind[name] = per_kind.get(name, 0.0) + span
        wait = min(span, max(0.0, t.get("exchange_ns", 0.0) + t.get("handoff_ns", 0.0)))
        if name in ("qkv", "o_proj", "gate_up", "down"):
            cats["wait_ns"] += wait
            cats["weight_gemv_ns"] += span - wait
        elif name == "attention":
            cats["wait_ns"] += wait
            cats["attention_ns"] += span - wait
        elif name in ("lm_head", "argmax"):
            cats["wait_ns"] += wait
            cats["lm_head_ns"] += span - wait
        else:
            cats["other_ns"] += span
    step_ns = max((t["end_ns"] for t in tab.values()), default=0.0)
    return {"step_ns": step_ns, **{k: round(v, 1) for k, v in cats.items()},
            "per_phase_kind_ns": {k: round(v, 1) for k, v in per_kind.items()}}
