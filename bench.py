"""Benchmark: batch-1 decode steps/s of the megakernel on a Llama-3.2-1B-shaped model.

One "step" is one full decode step (every layer, attention over the cache, LM head and
argmax) for one token, run as one kernel launch.  Default workload: Llama-3.2-1B shape,
KV context 128, seeded synthetic bf16 weights, the step repeated at the same position
(its K/V write is idempotent).  Inputs are resident in HBM before timing starts.

Prints one JSON line (rank 0).  Other workloads (--workload) are for the design notes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOADS = {
    # name: (model shape, KV context / first position, greedy steps per timed step)
    "llama1b_ctx128": ("llama1b", 128),
    "llama1b_ctx8192": ("llama1b", 8192),
    "llama1b_greedy_from_1024": ("llama1b", 1024),
    "llama8b_ctx2048": ("llama8b", 2048),
}
METRIC = "batch-1 decode steps/sec (Llama-3.2-1B shape); achieved HBM GB/s vs peak"


def stored_traffic(workload: str, n_launch_bytes: float):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they were taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    from transformer_megakernel_amd.profile_summary import kernel_source_hash
    t = json.load(open(path))
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (lscpu's "Model name", read from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, W, kv, tok, pos, budget_s=20.0):
    """The CPU oracle (NumPy fp32, untuned) on this host, on a bounded sample of steps."""
    import numpy as np

    import oracle
    threads = os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count())
    Wn = W.as_numpy_bits()
    kvn = kv.detach().cpu().view(__import__("torch").int16).numpy().view(np.uint16).copy()
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_step(shape, Wn, kvn, tok, pos)
        n += 1
        el = time.perf_counter() - t0
        if el > budget_s or n >= 8:
            break
    return dict(value=round(n / el, 4), unit="steps/s", cores=int(threads), kind="oracle",
                sample=f"{n} decode steps of the same workload (NumPy fp32 oracle, {el:.1f} s)",
                cpu_model=cpu_model())


def copy_calibration(mib: int) -> None:
    """Three elementwise copies (dst = -src, int32) of ``mib`` MiB: per dispatch the HBM
    counters should read ``mib`` MiB fetched and ``mib`` MiB written."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty(n // 4, dtype=torch.int32, device="cuda:0")
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n}), flush=True)


def read_ceiling(mib: int) -> dict:
    """Plain streaming kernels for comparison, timed with events over 20 passes: the
    library's hand-written streaming read (mk_stream_read) over a sweep of launch shapes,
    torch's float32 sum over ``mib`` MiB (a read, a few bytes written) and an elementwise
    copy (``mib`` MiB read and written).  Prints and returns the median GB/s of each."""
    import torch

    from transformer_megakernel_amd import mk
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    out = torch.empty((), dtype=torch.float32, device="cuda:0")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")

    def timed(fn):
        for _ in range(3):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(21)]
        ev[0].record()
        for i in range(20):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(20))[10]

    sweep = {}
    for blocks in (256, 512, 1024, 2048, 4096, 8192):
        for unroll in (4, 8, 16):
            t = timed(lambda: mk.stream_read(src, sink, blocks, unroll))
            sweep[f"{blocks}x256 threads, {unroll} loads in flight"] = round(n / t / 1e6, 1)
    best = max(sweep, key=sweep.get)
    t_sum = timed(lambda: torch.sum(src, dim=0, out=out))
    t_copy = timed(lambda: dst.copy_(src))
    res = {"bytes": n, "stream_read_best_gb_per_s": sweep[best], "stream_read_best_shape": best,
           "stream_read_sweep_gb_per_s": sweep, "torch_sum_read_gb_per_s": round(n / t_sum / 1e6, 1),
           "torch_copy_read_plus_write_gb_per_s": round(2 * n / t_copy / 1e6, 1)}
    print(json.dumps(res), flush=True)
    return res


GEMV_VARIANTS = {0: "fp32 FMA on widened bf16 (the decode kernel)", 1: "v_dot2 bf16 pairs, activation hi+lo",
                 2: "MFMA 16x16x32 bf16, activation hi+mid+lo", 3: "LDS reads only"}


def gemv_page_bench(pages: int = 4000) -> dict:
    """Per-page cost of the step's matrix-vector work on one CU (4 waves, each over its own
    16 KiB page of 4 rows x 2048 bf16 in LDS, fp32 activation), per variant; plus each
    variant's first-page row sums against the fp32 FMA variant's."""
    import numpy as np
    import torch

    from transformer_megakernel_amd import mk
    blocks = 256
    res = {}
    rows = {}
    for v, name in GEMV_VARIANTS.items():
        ticks = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda:0")
        out = torch.zeros(blocks * 4 * 8, dtype=torch.float32, device="cuda:0")
        for rep in range(2):   # the first launch warms the code object
            mk.check(mk.lib().mk_bench_gemv_page(v, pages, blocks, mk.ptr(ticks), mk.ptr(out), None),
                     "mk_bench_gemv_page")
            torch.cuda.synchronize()
        t = ticks.cpu().numpy() * 0.01 / pages                 # us per page per wave (100 MHz ticks)
        rows[v] = out.cpu().numpy().reshape(blocks * 4, 8)[0, 4:8].astype(np.float64)
        res[name] = {"us_per_page_per_wave_median": round(float(np.median(t)), 4),
                     "us_per_page_per_wave_max": round(float(t.max()), 4)}
    for v in (1, 2):
        d = np.max(np.abs(rows[v] - rows[0])) / np.max(np.abs(rows[0]))
        res[GEMV_VARIANTS[v]]["max_rel_diff_vs_fp32_fma"] = float(f"{d:.3e}")
    fma = res[GEMV_VARIANTS[0]]["us_per_page_per_wave_median"]
    res["page"] = "16 KiB: 4 rows x 2048 bf16; 4 compute waves per CU, 256 CUs, 4000 pages each"
    res["stream_time_of_a_page_us"] = round(16384 * 256 / 8e12 * 1e6 / 4, 4)   # at 8 TB/s, per wave's share
    res["fma_vs_stream"] = round(fma / res["stream_time_of_a_page_us"], 3)
    print(json.dumps(res), flush=True)
    return res


def mall_bench() -> dict:
    """Does a buffer read moments ago come back faster (from the 256 MB memory-side cache)?
    Streams a 192 MiB buffer cold (after reading 2 GiB of other data), right after a
    non-temporal read of it, and right after a plain read of it; and checks whether a 2 GiB
    non-temporal stream in between evicts it."""
    import numpy as np
    import torch

    from transformer_megakernel_amd import mk
    mib = 192
    a = torch.ones((mib << 20) // 4, dtype=torch.float32, device="cuda:0")
    big = torch.ones((2048 << 20) // 4, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")

    def rd(t, unroll=8):
        mk.stream_read(t, sink, 256, unroll)

    def timed(t):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rd(t)
        e1.record()
        torch.cuda.synchronize()
        return round(a.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)

    res = {}
    for name, prep in [("cold", lambda: rd(big)), ("after a non-temporal read", lambda: (rd(big), rd(a))),
                       ("after a plain read", lambda: (rd(big), rd(a, -8))),
                       ("plain read, then 2 GiB non-temporal stream", lambda: (rd(big), rd(a, -8), rd(big))),
                       ("plain read, then 2 GiB plain stream", lambda: (rd(big), rd(a, -8), rd(big, -8)))]:
        v = []
        for _ in range(5):
            prep()
            torch.cuda.synchronize()
            v.append(timed(a))
        res[name + " (GB/s)"] = float(np.median(v))
    print(json.dumps(res), flush=True)
    return res


def poll_bench() -> dict:
    """Dependency-poll round trip while every CU streams weights into LDS the way the
    decode step's loaders do (0-4 pages of 16 KiB in flight per loader wave, two loaders
    per CU), for a vector and a scalar probe; and the time for all CUs to read one 16 KiB
    vector of 64-bit words at once against each reading its own."""
    import numpy as np
    import torch

    from transformer_megakernel_amd import mk
    blocks, probes, region = 256, 40, 8 << 20
    buf = torch.ones(blocks * region // 4, dtype=torch.float32, device="cuda:0")
    words = torch.zeros(blocks * probes * 16, dtype=torch.int64, device="cuda:0")
    out = torch.zeros(blocks * (probes + 4), dtype=torch.int64, device="cuda:0")
    res = {"probe": "one 64-bit word per probe, ~1 us apart; loaders: 16 x 1 KiB LDS-direct loads per page"}
    for scalar in (0, 1):
        for depth in (0, 1, 2, 4):
            for _ in range(2):
                mk.check(mk.lib().mk_bench_poll_latency(mk.ptr(buf), region, mk.ptr(words), depth, scalar, probes,
                                                        blocks, mk.ptr(out), None), "mk_bench_poll_latency")
                torch.cuda.synchronize()
            o = out.cpu().numpy()
            t = o[:blocks * probes].reshape(blocks, probes)[:, 5:] * 0.01   # us; skip the start-up probes
            r = {"median_us": round(float(np.median(t)), 3), "p90_us": round(float(np.percentile(t, 90)), 3)}
            if depth:
                end = o[blocks * probes:blocks * (probes + 1)]
                pages = o[blocks * (probes + 1):blocks * (probes + 3)].reshape(blocks, 2).sum(axis=1)
                start = o[blocks * (probes + 3):blocks * (probes + 4)]
                span_s = (end.max() - start.min()) * 1e-8
                r["loaders_gb_per_s"] = round(float(pages.sum() * 16384 / span_s / 1e9), 1)
            res[f"{'scalar' if scalar else 'vector'} probe, {2 * depth} pages in flight per CU"] = r
    reps = 20
    vec = torch.ones(blocks * 2048, dtype=torch.int64, device="cuda:0")
    out2 = torch.zeros(blocks * reps, dtype=torch.int64, device="cuda:0")
    for shared in (1, 0):
        for _ in range(2):
            mk.check(mk.lib().mk_bench_bcast_read(mk.ptr(vec), shared, reps, blocks, mk.ptr(out2), None),
                     "mk_bench_bcast_read")
            torch.cuda.synchronize()
        t = out2.cpu().numpy().reshape(blocks, reps)[:, 2:] * 0.01
        res[f"16 KiB read by every CU, {'the same vector' if shared else 'each its own'}"] = {
            "median_us": round(float(np.median(t)), 3), "p90_us": round(float(np.percentile(t, 90)), 3)}
    print(json.dumps(res), flush=True)
    return res


def traced_breakdown(m, shape, step_fn, n_steps: int, path: str, title: str) -> None:
    """Run ``n_steps`` steps with the per-instruction trace on and write the time
    breakdown (transformer_megakernel_amd.trace_breakdown) to ``path``."""
    from transformer_megakernel_amd import trace_breakdown as tb
    buf = m.enable_trace()
    P = m.plan()
    traces = []
    for _ in range(n_steps):
        buf.zero_()
        step_fn()
        m.sync()
        traces.append(tb.reshape(buf.cpu().numpy(), P["n_cus"]))
    m.disable_trace()
    nch = max(int(r[7]) for r in P["records"] if r[0] == tb.DOWN)
    rep = tb.report(traces, P, shape.n_layers, nch, title)
    with open(path, "w") as f:
        f.write(rep + "\n")
    print(rep, file=sys.stderr, flush=True)


def per_op_baseline(shape, W, kv, tok, pos, steps, warmup):
    """A conventional decode step for comparison: one PyTorch kernel (or a few) per
    operation, bf16 weights and matrix-vector products (fp32 accumulation inside the
    library), fp32 residual stream, run eagerly and replayed from a HIP graph.  Returns
    its timings, and its logits and next token for a sanity check against the megakernel.
    It is a baseline only: nothing in the library uses it."""
    import torch
    import torch.nn.functional as F
    L, d, hd, hq, hkv = shape.n_layers, shape.hidden, shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    hpg, eps, dev = hq // hkv, shape.rms_eps, "cuda:0"
    bf = torch.bfloat16
    wqkv = [torch.cat([W.wq[l], W.wk[l], W.wv[l]], 0).contiguous() for l in range(L)]   # fused, as usual
    wgu = [torch.cat([W.w_gate[l], W.w_up[l]], 0).contiguous() for l in range(L)]
    half = hd // 2
    inv = torch.tensor([shape.rope_theta ** (-2.0 * i / hd) for i in range(half)], dtype=torch.float64)
    ang = pos * inv
    cos = torch.cos(ang).float().to(dev)
    sin = torch.sin(ang).float().to(dev)
    tok_t = torch.tensor([tok], dtype=torch.long, device=dev)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device=dev)
    nxt = torch.zeros((), dtype=torch.long, device=dev)

    def rms(x, g):
        return x * torch.rsqrt(x.pow(2).mean() + eps) * g.float()

    def rope(t):   # t: (heads, hd), rotate-half
        a, b = t[:, :half], t[:, half:]
        return torch.cat([a * cos - b * sin, b * cos + a * sin], dim=1)

    def step():
        x = W.embed.index_select(0, tok_t)[0].float()
        for l in range(L):
            qkv = torch.mv(wqkv[l], rms(x, W.attn_norm[l]).to(bf)).float()
            q = rope(qkv[: hq * hd].view(hq, hd))
            k = rope(qkv[hq * hd: (hq + hkv) * hd].view(hkv, hd))
            v = qkv[(hq + hkv) * hd:].view(hkv, hd)
            kv[l, 0, :, pos, :] = k.to(bf)
            kv[l, 1, :, pos, :] = v.to(bf)
            K = kv[l, 0, :, : pos + 1, :].contiguous()            # (hkv, P+1, hd)
            V = kv[l, 1, :, : pos + 1, :].contiguous()
            qg = q.view(hkv, hpg, hd).transpose(1, 2).contiguous().to(bf)   # (hkv, hd, hpg)
            s_ = torch.bmm(K, qg).float() * (1.0 / hd ** 0.5)     # (hkv, P+1, hpg)
            pr = torch.softmax(s_, dim=1).transpose(1, 2).contiguous().to(bf)   # (hkv, hpg, P+1)
            o = torch.bmm(pr, V).float().reshape(hq * hd)
            x = x + torch.mv(W.wo[l], o.to(bf)).float()
            gu = torch.mv(wgu[l], rms(x, W.mlp_norm[l]).to(bf)).float()
            a = F.silu(gu[: shape.ffn]) * gu[shape.ffn:]
            x = x + torch.mv(W.w_down[l], a.to(bf)).float()
        logits.copy_(torch.mv(W.lm_head, rms(x, W.final_norm).to(bf)).float())
        nxt.copy_(torch.argmax(logits))

    def timed(fn, n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record()
        for i in range(n):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n))
        return per[len(per) // 2]

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    eager_us = timed(step, steps)
    ref_logits, ref_tok = logits.clone(), int(nxt.item())
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    same = True
    for _ in range(3):   # replays must reproduce the eager result
        logits.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = same and bool(torch.equal(logits, ref_logits)) and int(nxt.item()) == ref_tok
    graph_us = timed(graph.replay, steps)
    # Five replays bracketed by a marker kernel (the library's streaming read over 4 KiB):
    # in a kernel trace of this run, the kernels between two markers are one step.
    from transformer_megakernel_amd import mk
    mbuf = torch.zeros(1024, dtype=torch.float32, device=dev)
    msink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(5):
        mk.stream_read(mbuf, msink, 1, 1)
        graph.replay()
    mk.stream_read(mbuf, msink, 1, 1)
    torch.cuda.synchronize()
    return {"eager_us": round(eager_us, 1), "graph_us": round(graph_us, 1), "graph_replays_match_eager": same,
            "token": ref_tok}, ref_logits


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama1b_ctx128", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-op-baseline", action="store_true",
                    help="also time a conventional per-operation decode step (PyTorch kernels, eager and "
                         "as a HIP graph) on the same inputs and report it beside the megakernel")
    ap.add_argument("--per-op-record", default="", metavar="PATH",
                    help="with --per-op-baseline: also write its results (and the oracle comparison) to PATH")
    ap.add_argument("--breakdown", default="", metavar="PATH",
                    help="after the timed steps, run 10 traced steps and write the time breakdown to PATH")
    ap.add_argument("--read-ceiling", type=int, default=0, metavar="MIB",
                    help="only time plain streaming kernels (the library's streaming read over a sweep of "
                         "launch shapes, torch sum, copy) over MIB MiB and exit")
    ap.add_argument("--gemv-page-bench", action="store_true",
                    help="only time one matrix-vector page per wave from LDS, per variant (fp32 FMA, v_dot2, "
                         "MFMA, LDS reads alone), and exit")
    ap.add_argument("--mall-bench", action="store_true",
                    help="only measure whether a just-read buffer is re-read faster (memory-side cache), and exit")
    ap.add_argument("--poll-bench", action="store_true",
                    help="only time a dependency poll's round trip under the loaders' weight stream, and a "
                         "16 KiB activation broadcast, then exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 3 times (a plain copy kernel of known "
                         "size, to calibrate the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.read_ceiling:
        read_ceiling(args.read_ceiling)
        return
    if args.gemv_page_bench:
        gemv_page_bench()
        return
    if args.poll_bench:
        poll_bench()
        return
    if args.mall_bench:
        mall_bench()
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for {args.gpus}); "
              "the decode megakernel has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from transformer_megakernel_amd import mk, roofline, synth

    model, ctx = WORKLOADS[args.workload]
    shape = synth.ModelShape.named(model)
    dev = "cuda:0"
    max_ctx = ctx + max(args.steps + args.warmup, 1) + 1
    print(f"[bench] {args.workload}: generating weights", file=sys.stderr, flush=True)
    W = synth.make_weights(shape, seed=0, device=dev)
    kv = synth.make_kv_cache(shape, max_ctx, ctx, seed=1, device=dev)
    tok = synth.make_token(shape, seed=2)
    m = mk.Megakernel(shape, max_ctx, 0)
    m.load_weights(W)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device=dev)
    nxt = torch.zeros(1, dtype=torch.int32, device=dev)
    tokbuf = torch.tensor([tok], dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    greedy = args.workload == "llama1b_greedy_from_1024"

    def step(i):
        if greedy:   # consecutive positions, token chained on the device
            m.decode_step_dev(tokbuf, ctx + i, kv, logits, tokbuf, stream)
        else:
            m.decode_step(tok, ctx, kv, logits, nxt, stream)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i if not greedy else 0)
    m.sync(stream)
    if greedy:   # restart the chain so the timed steps walk positions ctx .. ctx+steps-1
        tokbuf.fill_(tok)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    m.sync(stream)
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]) * 1e3   # us
    total_ms = ev[0].elapsed_time(ev[-1])
    ms_per_step = total_ms / args.steps
    pos_mid = ctx + (args.steps // 2 if greedy else 0)
    bytes_step = roofline.step_bytes(shape, pos_mid)["total"]
    avg_us = float(per.mean())
    achieved = bytes_step / (avg_us * 1e-6) / 1e9
    traffic = stored_traffic(args.workload, bytes_step)
    out = {
        "metric": METRIC,
        "value": round(1000.0 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": {
                "llama1b_ctx128": "Llama-3.2-1B-shaped batch-1 decode step, KV context 128",
                "llama1b_ctx8192": "Llama-3.2-1B-shaped batch-1 decode step, KV context 8192",
                "llama1b_greedy_from_1024": "Llama-3.2-1B-shaped greedy decode from context 1024, device-chained tokens",
                "llama8b_ctx2048": "Llama-3.1-8B-shaped batch-1 decode step, KV context 2048",
            }[args.workload],
            "layers": shape.n_layers, "hidden": shape.hidden, "heads_q_kv": [shape.n_q_heads, shape.n_kv_heads],
            "head_dim": shape.head_dim, "ffn": shape.ffn, "vocab": shape.vocab, "context": ctx,
            "weights": "bf16", "activations_accumulate": "fp32",
            "us_per_token": {"p50": round(float(np.percentile(per, 50)), 2),
                             "p90": round(float(np.percentile(per, 90)), 2),
                             "p99": round(float(np.percentile(per, 99)), 2),
                             "min": round(float(per.min()), 2), "max": round(float(per.max()), 2)},
            "algorithmic_bytes_per_step": bytes_step,
            "wall_s": round(wall, 4),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": roofline.MI355X_HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / roofline.MI355X_HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
    }
    if args.breakdown:
        print("[bench] traced steps for the time breakdown", file=sys.stderr, flush=True)
        traced_breakdown(m, shape, lambda: step(0), 10, args.breakdown,
                         f"Time breakdown: {out['config']['workload']} (bench.py --breakdown)")
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(shape, W, kv, tok, ctx)
    if args.per_op_baseline and not greedy:
        print("[bench] per-operation baseline", file=sys.stderr, flush=True)
        m.decode_step(tok, ctx, kv, logits, nxt, stream)
        m.sync(stream)
        mk_logits, mk_tok = logits.clone(), int(nxt.item())
        res, po_logits = per_op_baseline(shape, W, kv, tok, ctx, max(args.steps // 4, 10), 3)
        res["megakernel_us"] = round(float(np.percentile(per, 50)), 1)
        res["same_token_as_megakernel"] = res["token"] == mk_tok
        res["max_abs_logit_diff_vs_megakernel"] = round(float((po_logits - mk_logits).abs().max()), 4)
        # both against the oracle (the per-operation step rounds its activations to bf16
        # before each product, as such steps usually do; the megakernel keeps them fp32)
        import oracle
        kvn = kv.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy()
        ref, ref_tok = oracle.decode_step(shape, W.as_numpy_bits(), kvn, tok, ctx, return_next=True)
        for name, lg, t in (("per_op", po_logits, res["token"]), ("megakernel", mk_logits, mk_tok)):
            g = lg.cpu().numpy().astype(np.float64)
            res[f"{name}_vs_oracle"] = {
                "max_abs": round(float(np.max(np.abs(g - ref))), 5),
                "rel_l2": round(float(np.linalg.norm(g - ref) / np.linalg.norm(ref)), 6),
                "same_token": t == ref_tok}
        res["launches_and_gaps"] = ("from a kernel trace of this run: profile_summary per_op "
                                    "(kernels between the marker launches are one graph replay)")
        out["per_op_baseline"] = res
        if args.per_op_record:
            with open(args.per_op_record, "w") as f:
                json.dump(res, f, indent=1)
    m.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
