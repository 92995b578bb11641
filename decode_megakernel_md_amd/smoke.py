"""Smoke check: one small decode step on cuda:0 against the oracle."""
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
    w = WL.tiny_dense()
    m = DeviceModel(w)
    toks = synth.tokens(w, 1)
    pos = [w.context]
    g = GU.run_gpu_step(m, toks, pos)
    o, _ = GU.run_oracle_step(w, toks, pos)
    err = GU.compare_step(w, g, o, "smoke")
    print(f"smoke ok: {w.name} next={int(g['next'][0])} max|dlogit|/rms={err:.2e}")
