"""Driver for rocprofv3 counter runs.

    python -m decode_megakernel_md_amd.profile_run [--workload dense_27b] [--batch 1] [--steps 3]
                                                    [--multilaunch | --compare] [--copy-mib 1024]
                                                    [--max-batch 64] [--verify]

First a plain device-to-device copy of --copy-mib MiB (its byte count is
known, so HBM counters read for it calibrate the counters read for the
decode step), then --steps decode steps of the workload at the given batch
and context, greedy tokens chained on the device.  --compare runs the steps
once as the megakernel and, after a pause of 20 ms, once as the multi-launch
baseline (one launch per phase), so that one kernel trace holds both.
--verify runs --steps verify launches (an anchor and 7 uniform random drafts of
sequence 0 at the workload's context) instead of decode steps."""
from __future__ import annotations

import argparse
import os
import sys
import time


def print_code_maps() -> None:
    """The executable mappings of this process (address range and file), so
    that the frames of any fault after this point can be attributed."""
    try:
        with open(f"/proc/{os.getpid()}/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and "x" in parts[1]:
                    print(f"# map {parts[0]} {parts[5]}", file=sys.stderr)
    except OSError as e:
        print(f"# maps unavailable: {e}", file=sys.stderr)
    sys.stderr.flush()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="dense_27b")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--multilaunch", action="store_true")
    ap.add_argument("--compare", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--max-batch", type=int, default=0, help="sequence slots (above 8: the 64-row kernel build)")
    ap.add_argument("--verify", action="store_true", help="verify launches (1 anchor + 7 drafts) instead of decode steps")
    args = ap.parse_args()
    import torch
    import synth
    from synth import workloads as WL
    from decode_megakernel_md_amd.model import DeviceModel

    dev = torch.device("cuda:0")
    n = args.copy_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    print(f"# calibration copy: {n} bytes read, {n} bytes written", flush=True)

    w = WL.get(args.workload)
    if args.max_batch:
        w = w.replace(name=w.name + f"_b{args.max_batch}", max_batch=args.max_batch)
    m = DeviceModel(w)
    B = args.batch
    toks = torch.empty((args.steps + 1, B), dtype=torch.int32, device=dev)
    toks[0] = torch.tensor(synth.tokens(w, B), device=dev)
    logits = torch.empty((B, w.vocab), dtype=torch.float32, device=dev)
    ids = None
    if w.is_moe:
        ids = torch.empty((w.n_layers, B, w.top_k), dtype=torch.int32, device=dev)
    if args.verify:
        import numpy as np
        n = 8
        vt = torch.tensor(np.random.default_rng(5).integers(0, w.vocab, size=(1, n)).astype(np.int32), device=dev)
        vp = torch.full((1,), w.context, dtype=torch.int32, device=dev)
        vlog = torch.empty((1, n, w.vocab), dtype=torch.float32, device=dev)
        acc = torch.empty((1,), dtype=torch.int32, device=dev)
        nxt = torch.empty((1,), dtype=torch.int32, device=dev)
        for s in range(args.steps):
            m.verify(vt, vp, vlog, acc, nxt)
        torch.cuda.synchronize()
        m.device_status()
        print(f"# {w.name}: {args.steps} verify launches of 1 + {n - 1} tokens", flush=True)
        del vt, vp, vlog, acc, nxt
    modes = [] if args.verify else ([False, True] if args.compare else [args.multilaunch])
    for ml in modes:
        for s in range(args.steps):
            pos = torch.full((B,), w.context + s, dtype=torch.int32, device=dev)
            m.decode(toks[s], pos, logits, toks[s + 1], ids, multilaunch=ml)
        torch.cuda.synchronize()
        m.device_status()
        print(f"# {w.name}: {args.steps} steps at batch {B} ({'multi-launch' if ml else 'megakernel'})", flush=True)
        time.sleep(0.02)
    # release every device object before returning, so that the runtime's
    # teardown at exit (which runs after the profiler has finalised) has
    # nothing of ours left to free
    m.close()
    del m, toks, logits, ids
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print_code_maps()
    print("# released", flush=True)


if __name__ == "__main__":
    sys.exit(main())
