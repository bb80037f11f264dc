"""The time-breakdown arithmetic on synthetic traces whose answer is known by construction
(no GPU): the per-CU category split and the per-layer critical-path segments."""
import numpy as np

from transformer_megakernel_amd import mk
from transformer_megakernel_amd import trace_breakdown as tb
from transformer_megakernel_amd.synth import ModelShape


def _plan(n_cus=4):
    s = ModelShape.named("tiny")
    return s, mk.Megakernel.plan_only(s, 64, n_cus).plan()


def test_categories_split_a_sequential_timeline_exactly():
    s, P = _plan()
    off = P["offsets"]
    L = int(max(np.diff(off)))
    tr = np.zeros((P["n_cus"], L, tb.SLOTS), np.int64)
    setup, poll, sync, stage, comp, wwait = 3, 40, 5, 12, 70, 25
    for cu in range(P["n_cus"]):
        t = 1000 + 17 * cu
        for i in range(int(off[cu + 1] - off[cu])):
            tr[cu, i, 0] = t
            tr[cu, i, 1] = t + setup
            tr[cu, i, 2] = t + setup + poll
            tr[cu, i, 3] = t + setup + poll + sync
            tr[cu, i, 4] = t + setup + poll + sync + stage
            tr[cu, i, 5] = tr[cu, i, 4]
            tr[cu, i, 6] = tr[cu, i, 5] + comp
            tr[cu, i, 7] = tr[cu, i, 6]
            tr[cu, i, 9] = tb.N_COMPUTE_WAVES * wwait
            t = tr[cu, i, 6]
    c = tb.categories(tr, P)
    n = np.diff(off).astype(float)
    per = lambda v: float(np.mean(n * v)) * tb.TICK_US
    assert np.isclose(c["dependency waits"], per(poll))
    assert np.isclose(c["inter-wave sync"], per(sync))
    assert np.isclose(c["activation staging"], per(stage))
    assert np.isclose(c["other"], per(setup))
    assert np.isclose(c["weight waits"], per(wwait))
    assert np.isclose(c["compute (matvec, attention)"], per(comp - wwait))
    assert np.isclose(sum(c[k] for k in tb.CATEGORIES), c["span (mean over CUs)"])


def test_layer_path_recovers_the_constructed_segments():
    s, P = _plan()
    off, rec = P["offsets"], P["records"]
    L = int(max(np.diff(off)))
    tr = np.zeros((P["n_cus"], L, tb.SLOTS), np.int64)
    seg = [30, 8, 45, 11, 20, 9, 60, 33, 14]          # ticks, in tb.SEGMENTS order
    nch = int(max(r[7] for r in rec if r[0] == tb.DOWN))
    layer_len = sum(seg)

    def phase_times(layer):
        b = np.cumsum([0] + seg) + 5000 + layer * layer_len
        return dict(x_in=b[0], qkv_done=b[1], a_in=b[2], a_done=b[3], o_in=b[4], o_done=b[5], g_in=b[6],
                    g_done=b[7], d_done=b[8])

    for cu in range(P["n_cus"]):
        for j, i in enumerate(range(int(off[cu]), int(off[cu + 1]))):
            op, layer, chunk = int(rec[i][0]), int(rec[i][1]), int(rec[i][6])
            if op == tb.LMHEAD:
                tr[cu, j, 2] = 5000 + s.n_layers * layer_len
                tr[cu, j, 6] = tr[cu, j, 7] = tr[cu, j, 2] + 100 + cu
                continue
            T = phase_times(layer)
            if op == tb.QKV:
                tr[cu, j, 2], tr[cu, j, 6] = T["x_in"], T["qkv_done"] - cu      # slowest CU: cu 0
            elif op == tb.ATTN:
                tr[cu, j, 2], tr[cu, j, 7] = T["a_in"], T["a_done"]
            elif op == tb.O:
                tr[cu, j, 2], tr[cu, j, 6] = T["o_in"], T["o_done"]
            elif op == tb.GATEUP:
                tr[cu, j, 2], tr[cu, j, 6] = T["g_in"], T["g_done"]
            elif op == tb.DOWN:
                tr[cu, j, 6] = T["d_done"] if chunk == nch - 1 else T["g_done"] + 1
    # leader start marks (the report's span needs them): just before each instruction
    first = np.where(tr[..., 2] > 0, tr[..., 2], np.maximum(tr[..., 6], tr[..., 7])) - 1
    tr[..., 0] = np.where(first > 0, first, 0)
    idx = tb.plan_index(P, L)
    path = tb.layer_path(tr, idx, s.n_layers, nch)
    assert np.allclose(path, np.array(seg) * tb.TICK_US)
    lm = tb.lm_head(tr, idx, s.n_layers)
    assert np.isclose(lm["slowest CU done"], (100 + P["n_cus"] - 1) * tb.TICK_US)
    rep = tb.report([tr], P, s.n_layers, nch, "synthetic")
    assert "hop attention -> O" in rep and "weight waits" in rep
