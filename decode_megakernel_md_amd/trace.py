"""In-kernel phase trace: record per-workgroup wall-clock stamps around every
sync point of a step (md_set_trace) and summarise phase and wait times.

    python -m decode_megakernel_md_amd.trace [--workload dense_27b] [--batches 1,8] [--max-batch 64] [--dump PREFIX]

prints, per phase kind, the median and slowest workgroup's time per layer,
the release latency of its sync point (last arrival to median wait end) and
the medians of the phase's own sub-stamps: the end of the wait to stamp 0
(weight-streaming phases: the stream starts; attention: q is ready), and
stamp 0 to stamps 1, 2, 3 (streams: 2 = stream done; attention: 3 = this
workgroup's blocks done, 1 = its partial stored, 2 = combine done); and,
measured from the workgroup's arrival at the previous sync point, when its
previous phase's stores had completed (its arrival made), when its slot
tables were built and when it started to wait (after the prefetch)."""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import check, lib


def phase_names(w, verify=False):
    """Names of the phases of one step, in sync-point order."""
    names = ["embed"]
    for l in range(w.n_layers):
        kind = w.layer_kind(l)
        if kind == "gqa":
            names += ["qkv"] + (["kv_write"] if verify else []) + ["attn", "oproj"]
        elif kind == "kda":
            names += ["kda_proj", "kda_rec", "kda_o"]
        else:
            names += ["mla_a", "mla_b", "mla_absorb", "mla_attn", "mla_out", "mla_o"]
        names += ["moe_a", "moe_b", "moe_down"] if w.is_moe else ["gateup", "down"]
    names += ["lmhead"]
    return names


class Tracer:
    def __init__(self, model, n_sync_max=2048):
        import torch
        self.m = model
        self.G = lib().md_grid_size(model.handle)
        self.n = max(2 * n_sync_max + 1, 16384)
        self.buf = torch.zeros((self.G, self.n), dtype=torch.int64, device=model.device)
        check(lib().md_set_trace(model.handle, ctypes.c_void_p(self.buf.data_ptr()), self.n))

    def stop(self):
        check(lib().md_set_trace(self.m.handle, None, 0))

    def summary(self, names, rate_hz=100e6):
        """Per phase kind (summed over its layers, microseconds): median and
        slowest workgroup's work time, the release latency of its sync point
        (last arrival -> median wait end), and medians of its sub-stamps."""
        t = self.buf.cpu().numpy().astype(np.float64) / rate_hz * 1e6
        raw = self.buf.cpu().numpy()
        start = t[:, -1]
        ns = len(names)
        work = np.empty((self.G, ns))
        prev = start
        release = np.empty(ns)
        for s in range(ns):
            end = t[:, 2 * s]
            work[:, s] = end - prev
            wait_end = t[:, 2 * s + 1]
            # the last sync point of a decode step has no wait (its last
            # arrival reduces the argmax)
            release[s] = np.median(wait_end) - end.max() if np.all(raw[:, 2 * s + 1] > 0) else 0.0
            prev = wait_end
        total = t[:, 2 * (ns - 1)].max() - start.min()
        h = self.n // 2
        sub = t[:, h: h + 8 * ns].reshape(self.G, ns, 8)
        subraw = raw[:, h: h + 8 * ns].reshape(self.G, ns, 8)
        out = {}
        # phase s waits on sync point s-1: its wait ends at t[2(s-1)+1]; the
        # previous phase's work ends at t[2(s-1)]
        wait_ends = [start] + [t[:, 2 * s + 1] for s in range(ns - 1)]
        prev_ends = [start] + [t[:, 2 * s] for s in range(ns - 1)]
        keys = ("med", "max", "release", "to_s0", "s0_s1", "s0_s2", "s0_s3", "arr_done", "arr_built", "arr_wait")
        for s, nm in enumerate(names):
            d = out.setdefault(nm, dict({"n": 0}, **{k: 0.0 for k in keys}))
            d["n"] += 1
            d["med"] += float(np.median(work[:, s]))
            d["max"] += float(work[:, s].max())
            d["release"] += float(release[s])
            ok = lambda k: bool(np.all(subraw[:, s, k] > 0))  # noqa: E731
            if ok(0):
                d["to_s0"] += float(np.median(sub[:, s, 0] - wait_ends[s]))
                for k, key in ((1, "s0_s1"), (2, "s0_s2"), (3, "s0_s3")):
                    if ok(k):
                        d[key] += float(np.median(sub[:, s, k] - sub[:, s, 0]))
            if ok(6):
                d["arr_done"] += float(np.median(sub[:, s, 6] - prev_ends[s]))
            if ok(4):
                d["arr_built"] += float(np.median(sub[:, s, 4] - prev_ends[s]))
            if ok(5):
                d["arr_wait"] += float(np.median(sub[:, s, 5] - prev_ends[s]))
        return out, total


def main():
    import argparse
    import sys

    import torch

    import synth
    from synth import workloads as WL

    from .model import DeviceModel
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="dense_27b")
    ap.add_argument("--batches", default="1,8")
    ap.add_argument("--max-batch", type=int, default=0, help="sequence slots (above 8: the 64-row kernel build)")
    ap.add_argument("--dump", default="", help="also save every workgroup's stamps (100 MHz ticks from the first "
                    "workgroup's start, -1: not recorded) to DUMP_b<B>.npz")
    args = ap.parse_args()
    w = WL.get(args.workload)
    if args.max_batch:
        w = w.replace(max_batch=args.max_batch)
    m = DeviceModel(w)
    for B in [int(b) for b in args.batches.split(",")]:
        toks = torch.tensor(synth.tokens(w, B), device=m.device)
        pos = torch.full((B,), w.context, dtype=torch.int32, device=m.device)
        logits = torch.empty((B, w.vocab), device=m.device)
        nxt = torch.empty((B,), dtype=torch.int32, device=m.device)
        ids = torch.empty((w.n_layers, B, max(w.top_k, 1)), dtype=torch.int32, device=m.device)
        for _ in range(2):
            m.decode(toks, pos, logits, nxt, ids if w.is_moe else None)
        tr = Tracer(m)
        m.decode(toks, pos, logits, nxt, ids if w.is_moe else None)
        torch.cuda.synchronize()
        m.device_status()
        tr.stop()
        if args.dump:
            raw = tr.buf.cpu().numpy()
            ns = len(phase_names(w))
            h = tr.n // 2
            t0 = raw[:, -1].min()
            rel = lambda a: np.where(a > 0, a - t0, -1).astype(np.int32)  # noqa: E731
            np.savez_compressed(f"{args.dump}_b{B}.npz", main=rel(raw[:, : 2 * ns]),
                                sub=rel(raw[:, h: h + 8 * ns]), start=rel(raw[:, -1]), names=np.array(phase_names(w)))
        out, total = tr.summary(phase_names(w))
        print(f"{w.name} B={B}: step {total:.1f} us (per layer below, us)")
        print("| phase | layers | work (median WG) | work (slowest WG) | release | wait end -> stamp 0 | "
              "stamp 0 -> 1 | stamp 0 -> 2 | stamp 0 -> 3 | prev arrival -> stores done | prev arrival -> tables built | "
              "prev arrival -> wait |")
        print("|---|---|---|---|---|---|---|---|---|---|---|---|")
        for k, d in out.items():
            n = d["n"]
            print(f"| {k} | {n} | {d['med'] / n:.1f} | {d['max'] / n:.1f} | {d['release'] / n:.1f} | "
                  f"{d['to_s0'] / n:.1f} | {d['s0_s1'] / n:.1f} | {d['s0_s2'] / n:.1f} | {d['s0_s3'] / n:.1f} | "
                  f"{d['arr_done'] / n:.1f} | {d['arr_built'] / n:.1f} | {d['arr_wait'] / n:.1f} |")
        sys.stdout.flush()
        del tr
    m.close()


if __name__ == "__main__":
    main()
