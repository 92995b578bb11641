"""In-kernel phase trace: record per-workgroup wall-clock stamps around every
sync point of a step (md_set_trace) and summarise phase and wait times."""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import check, lib


def dense_phase_names(n_layers):
    names = ["embed"]
    for l in range(n_layers):
        names += ["qkv", "attn", "oproj", "gateup", "down"]
    names += ["lmhead"]
    return names


class Tracer:
    def __init__(self, model, n_sync_max=2048):
        import torch
        self.m = model
        self.G = lib().md_grid_size(model.handle)
        self.n = 2 * n_sync_max + 1
        self.n = 16384
        self.buf = torch.zeros((self.G, self.n), dtype=torch.int64, device=model.device)
        check(lib().md_set_trace(model.handle, ctypes.c_void_p(self.buf.data_ptr()), self.n))

    def stop(self):
        check(lib().md_set_trace(self.m.handle, None, 0))

    def summary(self, names, rate_hz=100e6):
        """Per phase kind: median/max work time across WGs and the release
        latency (last arrival -> median wait end), in microseconds."""
        t = self.buf.cpu().numpy().astype(np.float64) / rate_hz * 1e6
        start = t[:, -1]
        ns = len(names)
        work = np.empty((self.G, ns))
        prev = start
        release = np.empty(ns)
        for s in range(ns):
            end = t[:, 2 * s]
            work[:, s] = end - prev
            wait_end = t[:, 2 * s + 1]
            release[s] = np.median(wait_end) - end.max()
            prev = wait_end
        total = t[:, 2 * (ns - 1)].max() - start.min()
        # sub-phase stamps (GEMV phases): 0 slots built, 1 first group flushed, 2 sweep done
        sub = t[:, self.n // 2: self.n // 2 + 4 * ns].reshape(self.G, ns, 4)
        out = {}
        prevs = [start] + [t[:, 2 * s + 1] for s in range(ns - 1)]
        for s, nm in enumerate(names):
            d = out.setdefault(nm, {"n": 0, "med": 0.0, "max": 0.0, "release": 0.0, "to_slots": 0.0,
                                    "to_first": 0.0, "to_sweep_end": 0.0, "k3": 0.0})
            d["n"] += 1
            d["med"] += float(np.median(work[:, s]))
            d["max"] += float(work[:, s].max())
            d["release"] += float(release[s])
            if np.all(sub[:, s, 0] > 0):
                d["to_slots"] += float(np.median(sub[:, s, 0] - prevs[s]))
                d["to_first"] += float(np.median(sub[:, s, 1] - sub[:, s, 0]))
                d["to_sweep_end"] += float(np.median(sub[:, s, 2] - sub[:, s, 0]))
                if np.all(sub[:, s, 3] > 0):
                    d["k3"] += float(np.median(sub[:, s, 3] - sub[:, s, 0]))
        return out, total
