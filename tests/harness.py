"""Shared test helpers: draw a workload's inputs on the host and run the
oracle on them.  Inputs come from `synth` only."""
from __future__ import annotations

from typing import Dict, List

import numpy as np

import synth
from synth.workloads import Workload, kv_layout, tensor_inventory


class HostWeights:
    """Lazily drawn bf16 weights; keeps them if `cache` is set."""

    def __init__(self, w: Workload, cache: bool = True):
        self.w = w
        self.specs = {t.name: t for t in tensor_inventory(w)}
        self.cache = cache
        self._d: Dict[str, np.ndarray] = {}
        self.overrides: Dict[str, np.ndarray] = {}

    def __call__(self, name: str) -> np.ndarray:
        if name in self.overrides:
            return self.overrides[name]
        if name in self._d:
            return self._d[name]
        a = synth.weight_host(self.w, self.specs[name])
        if self.cache:
            self._d[name] = a
        return a

    def all(self) -> Dict[str, np.ndarray]:
        return {n: self(n) for n in self.specs}


def host_kv(w: Workload) -> List[np.ndarray]:
    return [synth.kv_layer_host(w, l) for l in range(w.n_layers)]


def kv_copy(kv: List[np.ndarray]) -> List[np.ndarray]:
    return [a.copy() for a in kv]


def zeros_like_weights(w: Workload, W: HostWeights, keep=("embed", "lm_head", "final_norm")):
    """Overrides that zero every layer matrix (norm gains stay)."""
    for t in tensor_inventory(w):
        if t.name in keep or t.kind == "gain":
            continue
        W.overrides[t.name] = np.zeros((t.rows, t.cols), dtype=np.uint16)
