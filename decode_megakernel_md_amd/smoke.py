"""Smoke check: small decode steps on cuda:0 against the oracle."""
from __future__ import annotations

import numpy as np


def run() -> None:
    import torch

    import synth
    from synth import workloads as WL
    from tests import gpu_util as GU

    from .model import DeviceModel

    if not torch.cuda.is_available():
        raise RuntimeError("smoke needs a GPU")
    # the tiny dense model, then a small hybrid one (MLA, delta rule, MoE) at batch 3
    for w, B in ((WL.tiny_dense(), 1), (WL.mini_hybrid(), 3)):
        m = DeviceModel(w)
        toks = synth.tokens(w, B)
        pos = [w.context - 2 * b for b in range(B)]
        g = GU.run_gpu_step(m, toks, pos)
        o, _ = GU.run_oracle_step(w, toks, pos)
        err = GU.compare_step(w, g, o, f"smoke {w.name}")
        m.close()
        print(f"smoke ok: {w.name} B={B} next={[int(t) for t in g['next']]} max|dlogit|/rms={err:.2e}")
