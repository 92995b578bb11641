"""Decode-step benchmark of the MI355X megakernel.

Workload: the 64-layer dense decoder shaped like a 27B model (hidden 5120,
GQA 40/8 x 128, SwiGLU 17408, vocab 152064), seeded synthetic bf16 weights,
context 4096, chained greedy decode steps (each step's argmax is the next
step's token, on the device; no host synchronisation inside the timed loop).
Batch 1 gives `value`; batch 8 is reported beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

Prints one JSON line.  `roofline.achieved` = algorithmic bytes of one step
(active weights + KV rows read) / mean duration of one megakernel launch,
timed with HIP events on the launch stream.  `extra` holds the hybrid MoE
model at batch 1 and 8, its verify step, paged-cache runs of both models and
both models with 64 sequence slots (the library's 64-row kernel build) at
batches of 16 to 64.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
METRIC = "decode tok/s + step latency at batch 1/8; achieved HBM GB/s vs 8 TB/s peak"


def algorithmic_bytes(w, B, positions_per_seq, expert_ids=None):
    """Bytes a decode step must read: every weight the step touches (layer
    matrices and norm gains -- of a MoE layer the router, the shared expert
    and the experts some token chose, taken from the step's reported expert
    ids -- the LM head, B embedding rows) plus every cached K/V or latent row
    attended (positions 0..pos inclusive) and every delta-rule state read."""
    import re
    from synth.workloads import tensor_inventory
    wb = 0
    expert = re.compile(r"^L(\d+)\.e(\d+)_")
    for t in tensor_inventory(w):
        if t.name == "embed":
            wb += B * t.cols * 2
            continue
        mt = expert.match(t.name)
        if mt:
            if expert_ids is None:
                raise ValueError("MoE byte count needs the step's expert ids")
            l, e = int(mt.group(1)), int(mt.group(2))
            if np.any(expert_ids[l, :B] == e):
                wb += t.numel * 2
            continue
        wb += t.numel * 2
    kvb = 0
    for l in range(w.n_layers):
        kind = w.layer_kind(l)
        for p in positions_per_seq:
            if kind == "gqa":
                kvb += 2 * w.n_kv_heads * w.head_dim * (int(p) + 1) * 2
            elif kind == "mla":
                kvb += (w.kv_lora + w.rope_dim) * (int(p) + 1) * 2
            else:
                kvb += w.kda_heads * w.kda_dk * w.kda_dv * 4
    return wb, kvb


def traffic_bytes(workload, B):
    """HBM bytes (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter
    reads for a plain device copy) per megakernel launch, as recorded by
    `profiling traffic` from rocprofv3 counter runs; None when there is no
    record for this workload and batch or the kernel has changed since."""
    from decode_megakernel_md_amd.profiling import traffic_for
    rec = traffic_for(workload, B)
    return None if rec is None else rec["bytes"]


def time_steps(m, B, steps, warmup, multilaunch=False):
    import torch
    w = m.w
    dev = m.device
    stream = torch.cuda.current_stream(dev)
    import synth
    toks = torch.empty((steps + warmup + 1, B), dtype=torch.int32, device=dev)
    toks[0] = torch.tensor(synth.tokens(w, B), device=dev)
    base = w.context
    pos = torch.tensor([[base + s] * B for s in range(steps + warmup)], dtype=torch.int32, device=dev)
    logits = torch.empty((B, w.vocab), dtype=torch.float32, device=dev)
    ids = None
    if w.is_moe:
        ids = torch.full((steps + warmup, w.n_layers, B, w.top_k), -1, dtype=torch.int32, device=dev)
    # warmup (positions base .. base+warmup-1), then the timed chain restarts at base
    for s in range(warmup):
        m.decode(toks[s], pos[s], logits, toks[s + 1], ids[s] if ids is not None else None, multilaunch=multilaunch)
    torch.cuda.synchronize(dev)
    m.device_status()
    toks[0] = toks[warmup]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize(dev)
    ev[0].record(stream)
    for s in range(steps):
        m.decode(toks[s], pos[s], logits, toks[s + 1], ids[s] if ids is not None else None, multilaunch=multilaunch)
        ev[s + 1].record(stream)
    torch.cuda.synchronize(dev)
    m.device_status()
    per = np.array([ev[s].elapsed_time(ev[s + 1]) for s in range(steps)], dtype=np.float64)
    total = ev[0].elapsed_time(ev[steps])
    return per, total, pos[:steps].cpu().numpy(), (ids[:steps].cpu().numpy() if ids is not None else None)


def time_multilaunch_graph(m, B, reps=16):
    """The multi-launch step (one launch per phase) captured in a HIP graph
    and replayed: the launch-overhead-free form of the non-megakernel
    baseline.  A graph holds two consecutive steps, one per sync-counter bank
    (each step clears the other bank's counters for the next), so that
    replays chain like eager steps.  Every step reuses the same token and
    positions; each checked replay starts from the same cache and state as
    the eager reference pair (restored in between: delta-rule states advance
    with every step) and must give its logits bitwise, with eager steps
    between the replays.  Returns (ms per step, every checked replay equal)."""
    import torch
    import synth
    w, dev = m.w, m.device
    toks = torch.tensor(synth.tokens(w, B), dtype=torch.int32, device=dev)
    pos = torch.tensor([w.context] * B, dtype=torch.int32, device=dev)
    ref = torch.empty((B, w.vocab), dtype=torch.float32, device=dev)
    out = torch.empty_like(ref)
    ids = torch.empty((w.n_layers, B, w.top_k), dtype=torch.int32, device=dev) if w.is_moe else None

    def eager_pair(dst):
        m.decode(toks, pos, dst, None, ids, multilaunch=True)
        m.decode(toks, pos, dst, None, ids, multilaunch=True)

    kv0 = m.kv.clone()
    eager_pair(ref)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        eager_pair(out)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        eager_pair(out)
    torch.cuda.synchronize(dev)
    ok = True
    for _ in range(3):
        out.fill_(float("nan"))
        m.kv.copy_(kv0)
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        ok = ok and bool(torch.equal(out, ref))
        m.kv.copy_(kv0)
        again = torch.empty_like(ref)
        eager_pair(again)         # eager work between replays (an even number of steps)
        torch.cuda.synchronize(dev)
        ok = ok and bool(torch.equal(again, ref))
    m.device_status()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    m.device_status()
    ms = e0.elapsed_time(e1) / (2 * reps)
    m.kv.copy_(kv0)
    del g, kv0
    return ms, ok


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, layers=8, B=1, min_seconds=10.0, max_rounds=16):
    """Time the oracle on layers 0..layers-1 plus the final norm and LM head
    for one token at the workload's context, repeated until at least
    min_seconds of CPU work are timed (a bounded sample), and extrapolate the
    mean per-layer time to all layers."""
    import synth
    from oracle import lib as olib, ptr
    from oracle import step as ostep
    from tests.harness import HostWeights

    wsub = w.replace(n_layers=layers)
    W = HostWeights(wsub)
    for t in synth.tensor_inventory(wsub):
        W(t.name)  # draw before timing
    kv = [synth.kv_layer_host(wsub, l) for l in range(layers)]
    toks = synth.tokens(w, B)
    pos = np.array([w.context] * B)
    t_layers = t_head = 0.0
    rounds = 0
    while rounds < max_rounds and (t_layers + t_head) < min_seconds:
        t0 = time.perf_counter()
        xs = np.empty((B, w.hidden))
        for b in range(B):
            olib().orc_embed(w.hidden, ptr(W("embed")), int(toks[b]), ptr(xs[b]))
        for l in range(layers):  # rewrites the same cache rows every round
            ostep._layer(wsub, W, l, xs, pos, kv[l], B, None, None)
        t1 = time.perf_counter()
        logits = np.empty((B, w.vocab), dtype=np.float32)
        for b in range(B):
            olib().orc_head(w.hidden, w.vocab, w.rms_eps, ptr(W("final_norm")), ptr(W("lm_head")), ptr(xs[b]),
                            ptr(logits[b]))
        t2 = time.perf_counter()
        t_layers += t1 - t0
        t_head += t2 - t1
        rounds += 1
    t_step = t_layers / rounds / layers * w.n_layers + t_head / rounds
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": B / t_step, "unit": "tok/s", "cores": cores, "cpu": cpu_model(), "kind": "oracle",
            "sample": f"fp64 oracle, batch {B}, context {w.context}: layers 0-{layers - 1} plus final norm and LM head, "
                      f"{rounds} rounds ({t_layers + t_head:.1f} s of CPU work timed), mean per layer "
                      f"{t_layers / rounds / layers * 1e3:.1f} ms and head {t_head / rounds * 1e3:.1f} ms, "
                      f"extrapolated to {w.n_layers} layers ({t_step:.2f} s per step)"}


def decode_bench(w, batches, steps, warmup, multilaunch=True, block_table=None):
    """Chained greedy decode steps at each batch size; returns per-batch
    results (and multi-launch timings when built).  block_table: the page
    map of a paged workload (w.kv_page > 0)."""
    import torch
    from decode_megakernel_md_amd.model import DeviceModel
    t0 = time.time()
    m = DeviceModel(w, block_table=block_table)
    torch.cuda.synchronize()
    print(f"# {w.name}: model ready in {time.time() - t0:.1f} s ({m.weight_bytes / 1e9:.2f} GB weights)",
          file=sys.stderr, flush=True)
    res = {}
    for B in batches:
        per, total, pos, ids = time_steps(m, B, steps, warmup)
        wb, kvb = [], []
        for s in range(steps):
            a, b = algorithmic_bytes(w, B, pos[s], ids[s] if ids is not None else None)
            wb.append(a)
            kvb.append(b)
        mean_ms = float(per.mean())
        bytes_step = float(np.mean(np.array(wb) + np.array(kvb)))
        gbs = bytes_step / (mean_ms * 1e-3) / 1e9
        res[B] = {"tok_s": B * steps / (total * 1e-3), "ms_per_step": total / steps,
                  "p50_ms": float(np.percentile(per, 50)), "p90_ms": float(np.percentile(per, 90)),
                  "kernel_ms": mean_ms, "bytes_per_step": bytes_step, "weight_bytes": float(np.mean(wb)),
                  "kv_bytes": float(np.mean(kvb)), "achieved_gbs": gbs, "frac": gbs / PEAK_GBS}
        print(f"# {w.name} B={B}: {res[B]['ms_per_step']:.3f} ms/step, {res[B]['tok_s']:.1f} tok/s, {gbs:.0f} GB/s "
              f"({100 * gbs / PEAK_GBS:.1f}% of 8 TB/s)", file=sys.stderr, flush=True)
    ml = {}
    if multilaunch:
        for B in batches:
            try:
                n = min(steps, 16)
                per, total, pos, _ = time_steps(m, B, n, 1, multilaunch=True)
                ml[B] = {"ms_per_step": total / n, "tok_s": B * n / (total * 1e-3)}
                gms, gok = time_multilaunch_graph(m, B)
                ml[B]["graph_ms_per_step"] = gms
                ml[B]["graph_replays_equal_eager"] = gok
                print(f"# {w.name} B={B} multi-launch: {ml[B]['ms_per_step']:.3f} ms/step eager, {gms:.3f} ms/step "
                      f"as a HIP graph (replays equal eager: {gok})", file=sys.stderr, flush=True)
            except Exception as e:  # not built for this configuration
                ml[B] = {"error": str(e)[:160]}
    m.close()
    del m
    torch.cuda.empty_cache()
    return res, ml


def verify_bench(w, steps, accepts=(3, 6), n=8):
    """Speculative verify of 1 anchor + 7 drafts at context w.context.  For
    acceptance length a the drafts are the greedy continuation of the anchor
    for a-1 tokens (computed by decode steps on the device, after which the
    delta-rule states are restored), then a token that differs from the
    greedy one, then uniform random ids; each timed verify starts from the
    same state (restored outside the timed region) and must accept a tokens.
    Reports accepted tokens/s = a / verify latency."""
    import torch
    import synth
    from decode_megakernel_md_amd.model import DeviceModel
    m = DeviceModel(w)
    dev = m.device
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    p0 = w.context
    kda = [l for l in range(w.n_layers) if w.layer_kind(l) == "kda"]
    saved = {l: m.kv_layer(l)[0].clone() for l in kda}

    def restore():
        for l in kda:
            m.kv_layer(l)[0].copy_(saved[l])

    anchor = int(synth.tokens(w, 1)[0])
    out = {}
    lg1 = torch.empty((1, w.vocab), dtype=torch.float32, device=dev)
    nx1 = torch.empty((1,), dtype=torch.int32, device=dev)
    for a in accepts:
        restore()
        toks = [anchor]
        for j in range(min(a, n - 1)):
            m.decode(torch.tensor([toks[-1]], dtype=torch.int32, device=dev),
                     torch.tensor([p0 + j], dtype=torch.int32, device=dev), lg1, nx1)
            toks.append(int(nx1.cpu()[0]))
        restore()
        if a < n:
            toks[a] = (toks[a] + 1) % w.vocab
        rng = np.random.default_rng(5000 + a)
        while len(toks) < n:
            toks.append(int(rng.integers(0, w.vocab)))
        tt = torch.tensor([toks[:n]], dtype=torch.int32, device=dev)
        pp = torch.tensor([p0], dtype=torch.int32, device=dev)
        lg = torch.empty((1, n, w.vocab), dtype=torch.float32, device=dev)
        acc = torch.empty((1,), dtype=torch.int32, device=dev)
        nx = torch.empty((1,), dtype=torch.int32, device=dev)
        ids = torch.empty((steps, w.n_layers, n, max(w.top_k, 1)), dtype=torch.int32, device=dev)
        for _ in range(2):
            restore()
            m.verify(tt, pp, lg, acc, nx, ids[0])
        torch.cuda.synchronize()
        m.device_status()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        accs = []
        for s_ in range(steps):
            restore()
            ev[s_][0].record(stream)
            m.verify(tt, pp, lg, acc, nx, ids[s_])
            ev[s_][1].record(stream)
            accs.append(acc.clone())
        torch.cuda.synchronize()
        m.device_status()
        per = np.array([e0.elapsed_time(e1) for e0, e1 in ev], dtype=np.float64)
        got = sorted(set(int(x.cpu()[0]) for x in accs))
        restore()
        idsn = ids.cpu().numpy()
        wb = [algorithmic_bytes(w, n, [p0], idsn[s_])[0] for s_ in range(steps)]
        _, kvb = algorithmic_bytes(w, 1, [p0], idsn[0])
        mean_ms = float(per.mean())
        bytes_v = float(np.mean(wb)) + kvb
        gbs = bytes_v / (mean_ms * 1e-3) / 1e9
        out[a] = {"accepted": got, "ms_per_verify": mean_ms, "p90_ms": float(np.percentile(per, 90)),
                  "accepted_tok_s": a / (mean_ms * 1e-3), "bytes_per_verify": bytes_v, "achieved_gbs": gbs,
                  "frac": gbs / PEAK_GBS}
        print(f"# {w.name} a={a}: {mean_ms:.3f} ms/verify, accepted {got}, {a / (mean_ms * 1e-3):.1f} accepted tok/s, "
              f"{gbs:.0f} GB/s", file=sys.stderr, flush=True)
    m.close()
    del m
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense_27b")
    ap.add_argument("--batches", default="1,2,4,8")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-multilaunch", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the hybrid MoE decode and verify sections")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU: the multi-GPU path is designed, not built; "
                                   "run with --gpus 1"}))
        sys.exit(2)

    from synth import workloads as WL

    w = WL.get(args.workload)
    batches = [int(b) for b in args.batches.split(",")]
    steps = min(args.steps, w.max_ctx - w.context - args.warmup)
    res, ml = decode_bench(w, batches, steps, args.warmup, multilaunch=not args.no_multilaunch)
    extra = {}
    if not args.no_extra and args.workload == "dense_27b":
        wh = WL.hybrid_moe()
        hs = min(16, wh.max_ctx - wh.context - args.warmup)
        hres, hml = decode_bench(wh, [1, 8], hs, args.warmup, multilaunch=not args.no_multilaunch)
        extra[wh.name] = {"steps": hs, "batches": {str(B): hres[B] for B in hres},
                          "multilaunch": {str(B): hml[B] for B in hml},
                          "roofline": {str(B): {"bound": "hbm", "achieved": hres[B]["achieved_gbs"], "peak": PEAK_GBS,
                                                "unit": "GB/s", "frac": hres[B]["frac"],
                                                "traffic": traffic_bytes("hybrid_moe", B)} for B in hres}}
        wv = WL.verify_hybrid()
        extra[wv.name] = {"steps": 8, "verify": {str(a): r for a, r in verify_bench(wv, 8).items()},
                          "traffic": traffic_bytes("verify_hybrid", 8)}
        # paged attention caches: every sequence's pages scattered over a pool
        # in random order (the same bytes per step as the contiguous runs)
        for base, page in ((WL.dense_27b(), 128), (WL.hybrid_moe(), 32)):
            npp = base.max_ctx // page
            wp = base.replace(name=base.name + f"_paged{page}", kv_page=page, kv_pages=base.max_batch * npp + 64)
            bt = np.random.default_rng(1).permutation(wp.kv_pages)[:wp.max_batch * npp].reshape(wp.max_batch, npp)
            ps = min(16, wp.max_ctx - wp.context - args.warmup)
            pres, _ = decode_bench(wp, [1, 8], ps, args.warmup, multilaunch=False, block_table=bt.astype(np.int32))
            extra[wp.name] = {"steps": ps, "kv_page": page, "kv_pages": wp.kv_pages,
                              "batches": {str(B): pres[B] for B in pres}}
        # more than 8 sequences: models with 64 slots run on the 64-row build
        for base, bs in ((WL.dense_27b(), [16, 32, 64]), (WL.hybrid_moe(), [16, 64])):
            ww = base.replace(name=base.name + "_b64", max_batch=64)
            wsteps = min(8, ww.max_ctx - ww.context - args.warmup)
            wres, _ = decode_bench(ww, bs, wsteps, args.warmup, multilaunch=False)
            extra[ww.name] = {"steps": wsteps, "max_batch": 64, "batches": {str(B): wres[B] for B in wres},
                              "traffic": {str(B): traffic_bytes(base.name + "_b64", B) for B in wres}}
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, layers=w.mla_every if w.attn_kind == 1 else 8)
        print(f"# cpu oracle: {cpu['value']:.4f} tok/s on {cpu['cores']} threads", file=sys.stderr, flush=True)
    B0 = batches[0]
    r0 = res[B0]
    line = {
        "metric": METRIC,
        "value": r0["tok_s"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": r0["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded random-init weights of the named shapes, sigma 0.02 (Irwin-Hall(4) draws: "
                "mean and variance of N(0, sigma), tails bounded at 3.46 sigma); KV cache and states of unit variance",
        "config": {"workload": w.name, "batch": B0, "context": w.context, "layers": w.n_layers,
                   "hidden": w.hidden, "chained_greedy_steps": steps},
        "roofline": {"bound": "hbm", "achieved": r0["achieved_gbs"], "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": r0["frac"], "traffic": traffic_bytes(args.workload, B0)},
        "cpu_baseline": cpu,
        "batches": {str(B): res[B] for B in batches},
        "multilaunch": {str(B): ml[B] for B in ml},
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
