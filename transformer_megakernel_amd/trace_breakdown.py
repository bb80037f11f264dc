"""Time breakdown of one decode step from the kernel's per-instruction trace.

The Megakernel article splits one forward into where its time goes (section
"Megakernel: a fusion design from scratch", results paragraph): storing activations,
waiting for consistency and loading them; RMSNorm and matrix-vector work; waiting for
weights; synchronisation between warps; setup, parameters and page state.  This module
gives the same split for the MI355X kernel, from the timestamps ``mk_set_trace`` records
(100 MHz ticks, per CU and instruction: see include/mk.h), in two views:

* **categories** -- each CU's span (its leader's first mark to its last) is cut into
  the intervals where its compute waves work on an instruction and the gaps between
  them.  Inside an instruction, the time its compute waves waited for weight pages
  (slot 9, averaged over the waves) is *weight waits* and the rest *compute*.  A gap
  is attributed, by the leader's marks of the next instruction, to *dependency waits*
  (polling other CUs' results: the article's consistency waits), *activation staging*
  (RMSNorm / RoPE / bf16 K,V and writes into LDS), *inter-wave sync* (the leader waiting
  for the compute waves to release an activation slot), or *other* (instruction
  decode, parameter loads, the final argmax).  The per-CU figures are averaged.
* **critical path per layer** -- the phase boundaries of one layer: a phase starts when
  the median CU has its inputs and ends when its slowest CU is done, because every next
  phase reads all of its results.  Hops are the gaps between one phase's end and the
  next one's start.
* **HBM idle per CU** -- the ticks the loader waves spent blocked on a full page ring
  with nothing of their own in flight (slot 11, summed over the two loaders, so halved
  here), attributed to the instruction whose page was waiting for a slot: the account of
  when each CU's weight stream stops because its on-chip buffers are full.  With the
  first ring page's issue time (slot 10) it also shows how far ahead of staging each
  instruction's pages were fetched.

Plain NumPy; it reads only the trace and the plan.
"""
from __future__ import annotations

import numpy as np

TICK_US = 0.01          # s_memrealtime runs at 100 MHz
QKV, ATTN, O, GATEUP, DOWN, LMHEAD = 1, 2, 3, 4, 5, 6
N_COMPUTE_WAVES = 4
N_LOADERS = 2
SLOTS = 12              # marks per (CU, instruction)

CATEGORIES = ("dependency waits", "activation staging", "inter-wave sync", "compute (matvec, attention)",
              "weight waits", "other")


def reshape(trace_words, n_cus: int) -> np.ndarray:
    """The flat trace buffer as int64 [n_cus][instructions][SLOTS]."""
    t = np.asarray(trace_words).astype(np.int64)
    return t.reshape(n_cus, -1, SLOTS)


def _overlap(a0, a1, b0, b1):
    return max(0, min(a1, b1) - max(a0, b0))


def categories(tr: np.ndarray, plan: dict) -> dict:
    """Mean per-CU split of the step span into CATEGORIES, in microseconds."""
    off = plan["offsets"]
    n_cus = tr.shape[0]
    tot = {c: 0.0 for c in CATEGORIES}
    span = 0.0
    for cu in range(n_cus):
        n = int(off[cu + 1] - off[cu])
        t = tr[cu, :n]
        start = int(t[0, 0])
        end = int(max(t[:, 7].max(), t[:, 6].max()))
        span += end - start
        cur = start                                   # end of the previous compute interval
        acc = dict.fromkeys(CATEGORIES, 0)
        for i in range(n):
            c0, c1 = int(t[i, 5]), int(t[i, 6])
            if c0 == 0 or c1 == 0:
                continue
            gap0, gap1 = cur, max(cur, c0)
            g = gap1 - gap0
            dep = _overlap(gap0, gap1, t[i, 1], t[i, 2]) if t[i, 2] else 0
            sync = _overlap(gap0, gap1, t[i, 2], t[i, 3]) if t[i, 3] else 0
            stage = _overlap(gap0, gap1, t[i, 3], t[i, 4]) if t[i, 4] else 0
            acc["dependency waits"] += dep
            acc["inter-wave sync"] += sync
            acc["activation staging"] += stage
            acc["other"] += g - dep - sync - stage
            busy = max(0, c1 - max(c0, cur))
            ww = min(busy, int(t[i, 9]) // N_COMPUTE_WAVES)
            acc["weight waits"] += ww
            acc["compute (matvec, attention)"] += busy - ww
            cur = max(cur, c1)
        acc["other"] += max(0, end - cur)             # after the last instruction: argmax, epoch
        for k in CATEGORIES:
            tot[k] += acc[k]
    out = {k: v / n_cus * TICK_US for k, v in tot.items()}
    out["span (mean over CUs)"] = span / n_cus * TICK_US
    return out


def plan_index(plan: dict, n_instr: int) -> np.ndarray:
    """Opcode, layer and down-chunk index of every (CU, instruction) slot of the trace:
    int32 [3][n_cus][n_instr] (opcode 0 where a CU's list is shorter)."""
    off, rec = plan["offsets"], plan["records"]
    n_cus = len(off) - 1
    idx = np.zeros((3, n_cus, n_instr), np.int32)
    for cu in range(n_cus):
        r = rec[int(off[cu]):int(off[cu + 1])]
        idx[0, cu, :len(r)] = r[:, 0]
        idx[1, cu, :len(r)] = r[:, 1]
        idx[2, cu, :len(r)] = r[:, 6]
    return idx


def _marks(tr, idx, op, layer, slot, chunk=None):
    m = (idx[0] == op) & (idx[1] == layer)
    if chunk is not None:
        m &= idx[2] == chunk
    v = tr[..., slot][m]
    return v[v > 0]


SEGMENTS = ("QKV", "hop QKV -> attention", "attention (incl. merge)", "hop attention -> O", "O projection",
            "hop O -> gate/up", "gate/up", "down chunks after the last gate/up", "hop down -> next layer")


def layer_path(tr: np.ndarray, idx: np.ndarray, n_layers: int, nch: int) -> np.ndarray:
    """Per layer, the critical-path segments of SEGMENTS in microseconds: [n_layers][9]."""
    out = np.zeros((n_layers, len(SEGMENTS)))
    for l in range(n_layers):
        b = [np.median(_marks(tr, idx, QKV, l, 2)), _marks(tr, idx, QKV, l, 6).max(),
             np.median(_marks(tr, idx, ATTN, l, 2)), _marks(tr, idx, ATTN, l, 7).max(),
             np.median(_marks(tr, idx, O, l, 2)), _marks(tr, idx, O, l, 6).max(),
             np.median(_marks(tr, idx, GATEUP, l, 2)), _marks(tr, idx, GATEUP, l, 6).max(),
             _marks(tr, idx, DOWN, l, 6, chunk=nch - 1).max(),
             np.median(_marks(tr, idx, QKV, l + 1, 2)) if l + 1 < n_layers
             else np.median(_marks(tr, idx, LMHEAD, n_layers, 2))]
        out[l] = np.diff(np.array(b, dtype=np.float64)) * TICK_US
    return out


def lm_head(tr: np.ndarray, idx: np.ndarray, n_layers: int) -> dict:
    """LM-head phase: inputs present (median CU) to compute done, median and slowest CU."""
    x_in = np.median(_marks(tr, idx, LMHEAD, n_layers, 2))
    done = _marks(tr, idx, LMHEAD, n_layers, 6)
    fin = _marks(tr, idx, LMHEAD, n_layers, 7)
    return {"median CU done": (np.median(done) - x_in) * TICK_US, "slowest CU done": (done.max() - x_in) * TICK_US,
            "argmax done": (fin.max() - x_in) * TICK_US}


def _per_cu(tr, idx, op, layer, slot, chunk=None):
    """The mark of one phase per CU (0 where the CU has no such instruction)."""
    m = (idx[0] == op) & (idx[1] == layer)
    if chunk is not None:
        m &= idx[2] == chunk
    return np.where(m, tr[..., slot], 0).max(axis=1)


def mlp_timeline(tr: np.ndarray, idx: np.ndarray, layers, nch: int) -> np.ndarray:
    """Gate/up and each down chunk, in microseconds after the median CU has its gate/up
    inputs: rows [gate/up, down 0, ...], columns (inputs present, staged, first compute
    wave starts, last compute wave done) x (median CU, slowest CU); mean over ``layers``."""
    rows = []
    for l in layers:
        t0 = np.median(_marks(tr, idx, GATEUP, l, 2))
        tab = []
        for op, ch in [(GATEUP, None)] + [(DOWN, c) for c in range(nch)]:
            r = []
            for slot in (2, 4, 5, 6):
                v = _per_cu(tr, idx, op, l, slot, ch)
                v = v[v > 0]
                r += [np.median(v) - t0, v.max() - t0] if v.size else [np.nan, np.nan]
            tab.append(r)
        rows.append(tab)
    return np.mean(np.array(rows, dtype=np.float64), axis=0) * TICK_US


def slow_cus(tr: np.ndarray, idx: np.ndarray, layers, n_layers: int) -> dict:
    """When the CUs finish gate/up (mean over ``layers``) and the LM head, relative to the
    median CU: CUs holding an attention item vs the others, and per XCD (work-groups are
    dealt to the eight XCDs round-robin)."""
    n_cus = tr.shape[0]
    att = np.array([(((idx[0][c] == ATTN) & (_per_cu(tr, idx, ATTN, 0, 2)[c] > 0)).any()) for c in range(n_cus)])
    out = {}
    for name, op, lay in (("gate/up done", GATEUP, layers), ("LM head done", LMHEAD, [n_layers])):
        d = np.mean([_per_cu(tr, idx, op, l, 6) - np.median(_per_cu(tr, idx, op, l, 6)) for l in lay], axis=0)
        d = d * TICK_US
        out[name] = {"attention CUs (median)": float(np.median(d[att])) if att.any() else float("nan"),
                     "other CUs (median)": float(np.median(d[~att])),
                     "per XCD (median)": [round(float(np.median(d[x::8])), 2) for x in range(8)],
                     "slowest CU": int(np.argmax(d)), "slowest (us after median)": float(d.max())}
    return out


OP_ROWS = [("QKV", QKV, None), ("attention (active items)", ATTN, None), ("O projection", O, None),
           ("gate/up", GATEUP, None), ("down 0", DOWN, 0), ("down 1", DOWN, 1), ("down 2", DOWN, 2),
           ("down 3", DOWN, 3), ("LM head", LMHEAD, None)]
OP_COLS = ("poll", "slot wait", "staging", "to compute", "compute", "page waits", "leader after")


def per_op(tr: np.ndarray, idx: np.ndarray, layers, n_layers: int) -> dict:
    """Median over CUs (and ``layers``) of each instruction type's intervals, in us: the
    leader's poll (marks 1-2), waiting for a free activation slot (2-3), staging (3-4),
    compute wave 0 starting after the staging (4-5), the compute waves' span (5-6), their
    page waits (slot 9 / 4 waves) and the leader's work after staging (4 or 6 to 7: the
    attention merge, the argmax)."""
    out = {}
    for name, op, ch in OP_ROWS:
        m = idx[0] == op
        m &= np.isin(idx[1], [n_layers] if op == LMHEAD else list(layers))
        if ch is not None:
            m &= idx[2] == ch
        t = tr[m].astype(np.float64)
        if op == ATTN:
            t = t[t[:, 2] > 0]
        if not len(t):
            continue
        cols = [t[:, 2] - t[:, 1], t[:, 3] - t[:, 2], t[:, 4] - t[:, 3], np.maximum(0, t[:, 5] - t[:, 4]),
                t[:, 6] - t[:, 5], t[:, 9] / N_COMPUTE_WAVES, t[:, 7] - np.maximum(t[:, 4], t[:, 6] * (op in (ATTN, LMHEAD)))]
        out[name] = [float(np.median(c)) * TICK_US for c in cols]
    return out


def hbm_idle(tr: np.ndarray, idx: np.ndarray, layers, n_layers: int) -> dict:
    """Per CU and layer, microseconds the CU's loaders sat blocked on a full ring with
    nothing in flight (slot 11 / N_LOADERS), in total and by the instruction type whose
    page was waiting; median over CUs, mean over ``layers``.  Also per instruction type,
    how long before its staging (mark 4) the first of its ring pages was issued (mark
    10), median over CUs and layers (negative: issued after staging)."""
    idle = tr[..., 11].astype(np.float64) / N_LOADERS * TICK_US
    out = {"total": [], "by type": {}, "ahead": {}}
    names = [(n, op, ch) for n, op, ch in OP_ROWS if op != LMHEAD]
    for l in layers:
        m = idx[1] == l
        out["total"].append(float(np.median(np.where(m, idle, 0).sum(axis=1))))
    out["total"] = float(np.mean(out["total"]))
    for name, op, ch in names:
        m = (idx[0] == op) & np.isin(idx[1], list(layers))
        if ch is not None:
            m &= idx[2] == ch
        per_cu = np.where(m, idle, 0).sum(axis=1) / max(1, len(list(layers)))
        out["by type"][name] = float(np.median(per_cu))
        t = tr[m].astype(np.float64)
        t = t[(t[:, 10] > 0) & (t[:, 4] > 0)]
        out["ahead"][name] = float(np.median(t[:, 4] - t[:, 10])) * TICK_US if len(t) else float("nan")
    m = idx[0] == LMHEAD
    out["by type"]["LM head"] = float(np.median(np.where(m, idle, 0).sum(axis=1)))
    return out


def step_span(tr: np.ndarray) -> float:
    """First mark of any CU to the last mark of any CU, microseconds."""
    first = tr[:, 0, 0][tr[:, 0, 0] > 0].min()
    last = max(tr[:, :, 7].max(), tr[:, :, 6].max())
    return float(last - first) * TICK_US


def report(traces: list, plan: dict, n_layers: int, nch: int, title: str = "") -> str:
    """Text report averaged over several traced steps (each [n_cus][instr][SLOTS])."""
    idx = plan_index(plan, traces[0].shape[1])
    cats = [categories(t, plan) for t in traces]
    paths = [layer_path(t, idx, n_layers, nch) for t in traces]
    lms = [lm_head(t, idx, n_layers) for t in traces]
    spans = [step_span(t) for t in traces]
    lines = []
    if title:
        lines.append(title)
    lines.append(f"traced steps: {len(traces)}; step span (first to last mark) {np.mean(spans):.1f} us")
    lines.append("")
    lines.append("Where a CU's time goes (mean over CUs and steps; the article's categories):")
    keys = list(CATEGORIES) + ["span (mean over CUs)"]
    for k in keys:
        v = np.mean([c[k] for c in cats])
        share = v / np.mean([c["span (mean over CUs)"] for c in cats])
        lines.append(f"  {k:32s} {v:8.1f} us  {share:6.1%}")
    lines.append("")
    inner = slice(2, n_layers - 2) if n_layers > 6 else slice(0, n_layers)
    P = np.mean(paths, axis=0)
    lines.append(f"Critical path of one layer (us; mean over layers {inner.start}..{inner.stop - 1} and steps):")
    for j, name in enumerate(SEGMENTS):
        lines.append(f"  {name:36s} {P[inner, j].mean():7.2f}")
    lines.append(f"  {'layer total':36s} {P[inner].sum(axis=1).mean():7.2f}")
    lines.append("")
    lines.append("LM head (us after the median CU has its inputs):")
    for k in lms[0]:
        lines.append(f"  {k:36s} {np.mean([m[k] for m in lms]):7.2f}")
    lay = list(range(n_layers))[inner]
    T = np.mean([mlp_timeline(t, idx, lay, nch) for t in traces], axis=0)
    lines.append("")
    lines.append("Gate/up and down chunks (us after the median CU has its gate/up inputs; median CU / slowest CU):")
    lines.append(f"  {'':12s} {'inputs present':>16s} {'staged':>16s} {'compute starts':>16s} {'compute done':>16s}")
    for r, name in enumerate(["gate/up"] + [f"down {c}" for c in range(nch)]):
        cells = " ".join(f"{T[r, 2 * k]:7.2f} /{T[r, 2 * k + 1]:7.2f}" for k in range(4))
        lines.append(f"  {name:12s} {cells}")
    O_ = [per_op(t, idx, lay, n_layers) for t in traces]
    lines.append("")
    lines.append("Per instruction type (us, median over CUs, mean over layers and steps):")
    lines.append(f"  {'':26s}" + "".join(f"{c:>13s}" for c in OP_COLS))
    for name, _, _ in OP_ROWS:
        if name in O_[0]:
            v = np.mean([o[name] for o in O_], axis=0)
            lines.append(f"  {name:26s}" + "".join(f"{x:13.2f}" for x in v))
    H = [hbm_idle(t, idx, lay, n_layers) for t in traces]
    layer_us = P[inner].sum(axis=1).mean()
    lines.append("")
    lines.append(f"HBM idle per CU: its loaders blocked on a full page ring with nothing in flight (us per layer, "
                 f"median CU, mean over layers {inner.start}..{inner.stop - 1} and steps):")
    lines.append(f"  {'total':26s} {np.mean([h['total'] for h in H]):7.2f} of the layer's {layer_us:.2f}")
    lines.append("  by the instruction whose page waited for a slot:")
    for k in H[0]["by type"]:
        if k == "LM head":
            continue
        lines.append(f"    {k:24s} {np.mean([h['by type'][k] for h in H]):7.2f}")
    lines.append(f"  LM head (once per step)    {np.mean([h['by type']['LM head'] for h in H]):7.2f}")
    lines.append("  first ring page issued before the instruction was staged (us, median CU):")
    for k in H[0]["ahead"]:
        a = np.array([h["ahead"][k] for h in H], dtype=float)
        a = a[~np.isnan(a)]
        lines.append(f"    {k:24s} " + (f"{a.mean():7.2f}" if a.size else "      -"))
    S = [slow_cus(t, idx, lay, n_layers) for t in traces]
    lines.append("")
    lines.append("Finishing order (us after the median CU; mean over steps):")
    for k in S[0]:
        a = np.mean([x[k]["attention CUs (median)"] for x in S])
        o = np.mean([x[k]["other CUs (median)"] for x in S])
        xcd = np.mean([x[k]["per XCD (median)"] for x in S], axis=0)
        mx = np.mean([x[k]["slowest (us after median)"] for x in S])
        lines.append(f"  {k}: attention CUs {a:+.2f}, other CUs {o:+.2f}, slowest CU {mx:+.2f}; per XCD "
                     + " ".join(f"{v:+.2f}" for v in xcd))
    return "\n".join(lines)
