"""Host-side checks of the C ABI and the static scheduler (no GPU needed)."""
import ctypes

import numpy as np
import pytest

from transformer_megakernel_amd import mk
from transformer_megakernel_amd.synth import ModelShape

OPS = dict(QKV=1, ATTN=2, O=3, GATEUP=4, DOWN=5, LMHEAD=6)


def test_library_exports_every_declared_symbol():
    L = mk.lib()
    names = mk.header_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert b"gfx950" in L.mk_version()


def test_error_codes_without_a_usable_device():
    cfg = mk.make_config(ModelShape.named("tiny"), 64)
    h = ctypes.c_void_p()
    assert mk.lib().mk_create(None, 0, ctypes.byref(h)) == mk.MK_EINVAL
    bad = mk.make_config(ModelShape.named("tiny"), 64)
    bad.head_dim = 96
    assert mk.lib().mk_create(ctypes.byref(bad), 0, ctypes.byref(h)) == mk.MK_EINVAL
    assert b"head_dim" in mk.lib().mk_strerror(mk.MK_EINVAL)
    # a bad device index is rejected, whether or not a GPU is present
    rc = mk.lib().mk_create(ctypes.byref(cfg), 4096, ctypes.byref(h))
    assert rc in (mk.MK_EINVAL, mk.MK_EHIP)
    assert mk.lib().mk_decode_step(None, 0, 0, None, None, None, None) == mk.MK_EINVAL
    assert mk.lib().mk_sync(None, None) == mk.MK_EINVAL
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        assert isinstance(mk.lib().mk_strerror(code), bytes)


@pytest.mark.parametrize("field,value", [("n_q_heads", 3), ("n_kv_heads", 3), ("hidden", 96),
                                         ("ffn", 100), ("hidden", 8192), ("max_ctx", 0)])
def test_config_validation_rejects_unsupported_shapes(field, value):
    cfg = mk.make_config(ModelShape.named("tiny"), 64)
    setattr(cfg, field, value)
    h = ctypes.c_void_p()
    assert mk.lib().mk_plan_only(ctypes.byref(cfg), 256, ctypes.byref(h)) == mk.MK_EINVAL


def _split(n, parts, i):
    return n * i // parts, n * (i + 1) // parts


@pytest.mark.parametrize("name", ["tiny", "llama1b", "llama8b"])
@pytest.mark.parametrize("n_cus", [256, 240, 80])
def test_plan_partitions_every_matrix_exactly(name, n_cus):
    s = ModelShape.named(name)
    try:
        m = mk.Megakernel.plan_only(s, 4096, n_cus)
    except mk.MkError:
        assert n_cus == 80 and name == "llama8b"   # 4096 / 80 > 64 residual rows per CU
        return
    P = m.plan()
    off, rec = P["offsets"], P["records"]
    nq, nkv = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    nqkv = nq + 2 * nkv
    cover = {}
    feats = {}
    for cu in range(n_cus):
        lst = rec[off[cu]:off[cu + 1]]
        assert lst[-1, 0] == OPS["LMHEAD"]
        phase = [(r[1], r[0]) for r in lst]
        assert phase == sorted(phase), "list not in phase order"
        o_rows = None
        for r in lst:
            op, layer, r0, n, k0, kn, a, b = r[:8]
            cover.setdefault((op, layer, a if op == OPS["DOWN"] else 0), []).append((r0, n, k0, kn, a, b))
            if op == OPS["GATEUP"]:
                # features come a block of 2^a at a time: q -> r0 + (q // fb) * rs + q % fb,
                # a block being a page's features or (where every CU gets whole blocks per
                # down chunk) eight, one 64-byte line of link words
                fpp = max(1, P["page_bytes"] // (4 * s.hidden))
                fb = 1 << int(a)
                assert fb == fpp or (fb == 8 and fpp < 8), (fb, fpp)
                feats.setdefault(layer, []).extend(r0 + (q // fb) * int(r[10]) + q % fb for q in range(n))
            if op == OPS["QKV"]:
                assert (k0, kn) == (0, s.hidden)
            if op == OPS["O"]:
                # the staging loads one residual row of x per lane
                assert (k0, kn) == (0, nq) and 0 < n <= 64
                o_rows = (r0, n)
            if op == OPS["DOWN"]:
                assert (r0, n) == o_rows and kn == s.ffn // b and k0 == a * kn
    for l in range(s.n_layers):
        assert sorted(feats[l]) == list(range(s.ffn)), "gate/up features not an exact partition"
        for op, total in ((OPS["QKV"], nqkv), (OPS["O"], s.hidden)):
            rows = sorted((r0, n) for r0, n, *_ in cover[(op, l, 0)] if n > 0)
            pos = 0
            for r0, n in rows:
                assert r0 == pos
                pos += n
            assert pos == total
        nch = cover[(OPS["DOWN"], l, 0)][0][5]
        for k in range(nch):
            rows = sorted((r0, n) for r0, n, *_ in cover[(OPS["DOWN"], l, k)])
            assert sum(n for _, n in rows) == s.hidden
        items = sorted((a, b) for *_, a, b in cover[(OPS["ATTN"], l, 0)])
        assert items == [(g, t) for g in range(s.n_kv_heads) for t in range(P["s_max"])]
    lm = sorted((r0, n) for r0, n, *_ in cover[(OPS["LMHEAD"], s.n_layers, 0)])
    assert sum(n for _, n in lm) == s.vocab and len(lm) == n_cus
    pos = 0
    for r0, n in lm:   # contiguous blocks, no gaps or overlaps
        assert r0 == pos and n > 0
        pos += n
    # LM-head blocks are sized per XCD (work-groups are dealt to the 8 XCDs round-robin):
    # CUs on even XCDs get a few per cent more rows than those on odd ones
    per_cu = [int(rec[off[cu + 1] - 1][3]) for cu in range(n_cus)]
    if n_cus % 8 == 0:
        even = np.mean([per_cu[c] for c in range(n_cus) if c % 2 == 0])
        odd = np.mean([per_cu[c] for c in range(n_cus) if c % 2 == 1])
        assert even >= odd
        if s.vocab >= 100 * n_cus:   # rounding aside: 1.04 / 0.96
            assert 1.07 < even / odd < 1.10
    else:
        assert max(per_cu) - min(per_cu) <= 1
    assert P["lds_bytes"] <= 160 * 1024
    assert P["page_bytes"] * P["ring_pages"] <= 128 * 1024


@pytest.mark.parametrize("name", ["tiny", "llama1b", "llama8b"])
@pytest.mark.parametrize("pos", [0, 16, 128, 300, 1279, 8192])
def test_plan_has_no_deadlock_at_any_position(name, pos):
    """Discrete-event run of the per-CU lists with the device's dependency rules: every
    CU executes its list in order, an instruction runs once everything it reads exists."""
    from tests.plan_sim import simulate
    s = ModelShape.named(name)
    m = mk.Megakernel.plan_only(s, 8193, 256)
    done, steps = simulate(s, m.plan(), pos)
    assert done, f"deadlock after {steps} rounds"


def _drop(plan, cu, pred):
    """A copy of ``plan`` with the first record of CU ``cu`` matching ``pred`` removed."""
    off, rec = plan["offsets"].copy(), plan["records"]
    idx = next(i for i in range(off[cu], off[cu + 1]) if pred(rec[i]))
    out = dict(plan)
    out["records"] = np.delete(rec, idx, axis=0)
    out["offsets"] = np.where(np.arange(off.size) > cu, off - 1, off)
    return out


def _move_before(plan, cu, pred_moved, pred_anchor):
    """A copy of ``plan`` where CU ``cu``'s first record matching ``pred_moved`` is moved
    in front of its first record matching ``pred_anchor``."""
    off, rec = plan["offsets"], plan["records"].copy()
    lst = list(range(off[cu], off[cu + 1]))
    i = next(j for j in lst if pred_moved(rec[j]))
    a = next(j for j in lst if pred_anchor(rec[j]))
    assert a < i
    block = rec[off[cu]:off[cu + 1]].tolist()
    r = block.pop(i - off[cu])
    block.insert(a - off[cu], r)
    rec[off[cu]:off[cu + 1]] = np.array(block, dtype=rec.dtype)
    out = dict(plan)
    out["records"] = rec
    return out


@pytest.mark.parametrize("pos", [128, 1024])
def test_plan_simulator_reports_planted_deadlocks(pos):
    """The schedule simulator is only a deadlock check if it can fail: a plan missing one
    CU's QKV rows of a layer (attention then waits for them forever), and a plan where a
    CU consumes a down-projection chunk before producing its own gate/up features for it
    (a wait on work queued behind itself), must both be reported as stuck."""
    from tests.plan_sim import simulate
    s = ModelShape.named("llama1b")
    P = mk.Megakernel.plan_only(s, 8193, 256).plan()
    assert simulate(s, P, pos)[0]
    missing = _drop(P, 37, lambda r: r[0] == OPS["QKV"] and r[1] == 5)
    assert not simulate(s, missing, pos)[0]
    circular = _move_before(P, 11, lambda r: r[0] == OPS["DOWN"] and r[1] == 3 and r[6] == 0,
                            lambda r: r[0] == OPS["GATEUP"] and r[1] == 3)
    assert not simulate(s, circular, pos)[0]


@pytest.mark.parametrize("name,pos,splits", [
    ("llama1b", 0, 1), ("llama1b", 1, 1), ("llama1b", 128, 1), ("llama1b", 129, 2), ("llama1b", 256, 2),
    ("llama1b", 300, 3), ("llama1b", 1024, 8), ("llama1b", 1279, 10), ("llama1b", 8191, 32),
    ("llama1b", 8192, 32), ("llama8b", 256, 1), ("llama8b", 257, 2), ("llama8b", 2048, 8)])
def test_attention_splits_cover_the_cached_keys(name, pos, splits):
    """Keys 0..pos-1 are in the cache and split into runs of at least 128 keys at head_dim
    64 (256 at head_dim 128), a whole number of pages, at most one per CU of a KV head's
    share; the current key joins the last split, so no split ever holds it alone."""
    from tests.plan_sim import split_geometry
    s = ModelShape.named(name)
    P = mk.Megakernel.plan_only(s, 8193, 256).plan()
    assert P["s_max"] == 32
    assert split_geometry(s, P, pos) == splits
