"""CPU checks of the GPU-parity comparison helpers: fed the oracle's own
outputs they pass, and each planted difference (a row's greedy token, one
expert id of one row, a logit beyond the tolerance) makes them fail.  This
guards the parity tests against comparing the oracle with itself."""
import numpy as np
import pytest

import synth
from oracle import step as ostep
from synth import workloads as WL
from tests import gpu_util as GU
from tests.harness import HostWeights, host_kv


@pytest.fixture(scope="module")
def verify_case():
    w = WL.mini_moe().replace(n_layers=2)
    W = HostWeights(w)
    kv = host_kv(w)
    toks = [int(t) for t in synth.tokens(w, 1)] + [int(t) for t in synth.tokens(w.replace(seed_base=99), 5)]
    v = ostep.verify_step(w, W, np.array([toks]), np.array([w.context]), kv)
    return w, v


def _as_gpu(v):
    logits = v["logits"][0].copy()
    ids = v["expert_ids"][0].copy()   # [L][n][k], as md_verify_step writes
    return logits, ids, int(v["accept_len"][0]), int(v["next"][0])


def test_oracle_against_itself_passes(verify_case):
    w, v = verify_case
    logits, ids, acc, nxt = _as_gpu(v)
    GU.compare_verify(w, logits, ids, acc, nxt, v, "self")


def test_a_different_expert_in_one_row_fails(verify_case):
    w, v = verify_case
    logits, ids, acc, nxt = _as_gpu(v)
    row = ids[1, 3]
    row[0], row[1] = row[1], row[0]          # same experts, other order: still a different choice list
    with pytest.raises(AssertionError, match="expert selection differs at layer 1 token 3"):
        GU.compare_verify(w, logits, ids, acc, nxt, v, "case-e")


def test_a_different_greedy_token_in_one_row_fails():
    """A designed verify output: row 1's runner-up sits just under its top
    logit; moving it just over (far within the logit tolerance) changes that
    row's greedy token, which must fail the argmax check."""
    w = WL.mini_dense()
    rng = np.random.default_rng(3)
    ref = rng.normal(0, 1, size=(1, 2, 64)).astype(np.float32)
    ref[0, 1, 5], ref[0, 1, 7] = 4.0, 3.999
    v = {"logits": ref, "argmax": np.argmax(ref, axis=-1).astype(np.int32), "accept_len": np.array([1]),
         "next": np.array([int(np.argmax(ref[0, 0]))])}
    GU.compare_verify(w, ref[0].copy(), None, 1, int(v["next"][0]), v, "case-same")
    got = ref[0].copy()
    got[1, 7] = 4.001
    with pytest.raises(AssertionError, match=r"b=1: argmax 7 != oracle 5"):
        GU.compare_verify(w, got, None, 1, int(v["next"][0]), v, "case-t")


def test_a_logit_beyond_tolerance_fails(verify_case):
    w, v = verify_case
    logits, ids, acc, nxt = _as_gpu(v)
    r = 5
    rms = float(np.sqrt(np.mean(v["logits"][0, r].astype(np.float64) ** 2)))
    low = int(np.argmin(logits[r]))
    logits[r, low] -= 3 * GU.LOGIT_TOL * rms
    with pytest.raises(AssertionError, match=r"b=5: max\|dlogit\|"):
        GU.compare_verify(w, logits, ids, acc, nxt, v, "case-l")


def test_router_margins_brute_force():
    lg = np.array([[0.5, 3.0, 1.0, 2.0]], dtype=np.float32)
    m = GU.router_margins(lg, 2)
    assert np.isclose(m[0], (2.0 - 1.0) / np.std(lg[0].astype(np.float64)))
    assert np.isinf(GU.router_margins(lg, 4)[0])
