"""CPU discrete-event run of a static schedule, with the device's dependency rules.

Each CU executes its instruction list strictly in order.  An instruction may run only
when every value it reads has been produced:

* QKV(l) reads all of x after layer l-1 (the embedding row for l = 0);
* ATTN(l, g, s), if split s is active at this position, reads q/k/v of KV head g and
  publishes its partial; with one active split, items s < heads per group each publish
  the attention output of query head g * hpg + s;
  a CU whose split index s is below the heads per group then merges head s of group g
  from all active splits (only when there is more than one split);
* O(l) reads every head's attention output; GATEUP(l) reads all of x after O(l);
* DOWN(l, k) reads chunk k of SiLU(gate)*up; its last chunk writes x rows;
* LMHEAD reads all of x after the last layer.

Returns (all lists finished, rounds taken).
"""
from __future__ import annotations

import math
from collections import defaultdict

QKV, ATTN, O, GATEUP, DOWN, LMHEAD = 1, 2, 3, 4, 5, 6


def split_geometry(shape, plan, pos):
    ppp = plan["page_bytes"] // (4 * shape.head_dim)
    nk = max(pos, 1)   # the cached keys 0..pos-1 (the current key joins the last split)
    min_chunk = 128 if shape.head_dim == 64 else 256   # the host plan's fewest keys per split
    chunk = max(min_chunk, math.ceil(nk / plan["s_max"]))
    chunk = math.ceil(chunk / ppp) * ppp
    return math.ceil(nk / chunk)


def simulate(shape, plan, pos):
    s_eff = split_geometry(shape, plan, pos)
    hd, hq, hkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    hpg = hq // hkv
    nq, nkv = hq * hd, hkv * hd
    off, rec = plan["offsets"], plan["records"]
    n_cus = plan["n_cus"]
    F, d = shape.ffn, shape.hidden

    x_rows = defaultdict(int)          # version -> rows written
    x_rows[0] = d                      # the embedding row exists from the start
    qkv_rows = defaultdict(int)        # (layer, group) -> rows written
    partials = defaultdict(set)        # (layer, group) -> splits published
    o_heads = defaultdict(set)         # layer -> heads written
    a_rows = defaultdict(int)          # (layer, chunk) -> rows written
    merged = set()                     # (cu, instr index) items published
    nch = max([int(r[7]) for r in rec if int(r[0]) == DOWN] or [1])
    csz = F // nch

    def group_of_qkv_row(r):
        if r < nq:
            return (r // hd) // hpg
        if r < nq + nkv:
            return (r - nq) // hd
        return (r - nq - nkv) // hd

    ptr = [int(off[c]) for c in range(n_cus)]
    end = [int(off[c + 1]) for c in range(n_cus)]
    rounds = 0
    progress = True
    while progress:
        progress = False
        rounds += 1
        for c in range(n_cus):
            while ptr[c] < end[c]:
                op, layer, r0, n, k0, kn, a, b = (int(v) for v in rec[ptr[c]][:8])
                if op == QKV:
                    if x_rows[2 * layer] < d:
                        break
                    for r in range(r0, r0 + n):
                        qkv_rows[(layer, group_of_qkv_row(r))] += 1
                elif op == ATTN:
                    g, s = a, b
                    key = (c, ptr[c])
                    active = s < hpg if s_eff == 1 else s < s_eff
                    if active and key not in merged:
                        if qkv_rows[(layer, g)] < (hpg + 2) * hd:
                            break
                        if s_eff == 1:
                            # one split: item (g, s < hpg) computes query head g * hpg + s
                            o_heads[layer].add(g * hpg + s)
                        else:
                            partials[(layer, g)].add(s)
                        merged.add(key)
                    if s_eff > 1 and s < hpg:
                        if len(partials[(layer, g)]) < s_eff:
                            break
                        o_heads[layer].add(g * hpg + s)
                elif op == O:
                    if len(o_heads[layer]) < hq:
                        break
                    x_rows[2 * layer + 1] += n
                elif op == GATEUP:
                    if x_rows[2 * layer + 1] < d:
                        break
                    rs = int(rec[ptr[c]][10])
                    fb = 1 << a                    # features per block (log2 in field a)
                    for q in range(n):
                        f = r0 + (q // fb) * rs + q % fb
                        a_rows[(layer, f // csz)] += 1
                elif op == DOWN:
                    if a_rows[(layer, a)] < kn:
                        break
                    if a == b - 1:
                        x_rows[2 * layer + 2] += n
                elif op == LMHEAD:
                    if x_rows[2 * shape.n_layers] < d:
                        break
                ptr[c] += 1
                progress = True
    return all(ptr[c] == end[c] for c in range(n_cus)), rounds
