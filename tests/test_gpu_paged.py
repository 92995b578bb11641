"""GPU: paged attention caches (md_decode_step_paged, md_verify_step_paged,
md_kv_copy_pages, md_kv_copy_slot) through the C ABI.

The oracle knows nothing of pages: it runs on the contiguous cache of every
sequence.  The paged model holds the same seeded cache scattered into the
pages of a block table (a random permutation of a pool with spare pages,
which are filled with NaN so that a read of a wrong page shows in the
logits), and its new rows are gathered back through the table for the
comparison.  Kimi K3 post, section "Future work" (KV cache movement and
management for agentic workloads)."""
import ctypes

import numpy as np
import pytest

import synth
from synth import workloads as WL
from tests import gpu_util as GU

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def paged(w, page, spare=3):
    """w with a paged cache of `page` positions: max_ctx rounded up to whole
    pages, a pool of every slot's pages plus `spare` unused ones."""
    C = (w.max_ctx + page - 1) // page * page
    return w.replace(name=w.name + f"_paged{page}", max_ctx=C, kv_page=page,
                     kv_pages=w.max_batch * (C // page) + spare)


def shuffled_table(w, seed):
    """Block table: slot s, page j -> a distinct page of the pool, in random order."""
    npp = w.max_ctx // w.kv_page
    perm = np.random.default_rng(seed).permutation(w.kv_pages)[:w.max_batch * npp]
    return perm.reshape(w.max_batch, npp).astype(np.int32)


def _model(w, bt=None):
    from decode_megakernel_md_amd.model import DeviceModel
    return DeviceModel(w, block_table=bt)


@pytest.mark.parametrize("name,page,B", [("mini_dense", 32, 3), ("mini_dense", 64, 8), ("mini_moe", 32, 5),
                                         ("mini_hybrid", 32, 3), ("mini_hybrid", 32, 8), ("mini_hybrid", 64, 8)])
def test_paged_decode_matches_oracle(torch_cuda, name, page, B):
    """(mini_hybrid, 32, 8): its MLA chunks are not page-aligned, so some
    partial 32-row blocks straddle a page boundary."""
    w = paged(WL.get(name), page)
    m = _model(w, shuffled_table(w, 7 + B))
    toks = synth.tokens(w, B)
    # ragged positions, some on a page's first row, some on its last
    pos = [min(w.context + 5 * b, w.max_ctx - 1) if b % 2 == 0 else max(w.context - 7 * b, 0) for b in range(B)]
    pos[-1] = page - 1 if B > 1 else pos[-1]
    print(f"case {w.name} B={B} pos={pos}", flush=True)
    g = GU.run_gpu_step(m, toks, pos)
    o, kv_ref = GU.run_oracle_step(w, toks, pos)
    err = GU.compare_step(w, g, o, f"{w.name} B={B}")
    GU.compare_kv_rows(w, m.kv_host(), kv_ref, pos, B)
    print(f"  max|dlogit|/rms = {err:.2e}")
    m.close()


@pytest.mark.parametrize("name,page,B", [("dense_27b", 128, 8), ("hybrid_moe", 32, 2)])
def test_paged_full_shape_layers_match_oracle(torch_cuda, name, page, B):
    """The two large models at full width and context (4 layers; the hybrid
    model's 4th is MLA over 8192 positions), paged, in bench.py's launch
    configuration."""
    w = paged(WL.get(name).replace(n_layers=4), page)
    toks = synth.tokens(w, B)
    pos = [w.context - 97 * b for b in range(B)]
    print(f"case {w.name} 4 layers B={B} pos={pos}", flush=True)
    m = _model(w, shuffled_table(w, 3))
    g = GU.run_gpu_step(m, toks, pos)
    o, kv_ref = GU.run_oracle_step(w, toks, pos)
    err = GU.compare_step(w, g, o, f"{w.name} B={B}")
    GU.compare_kv_rows(w, m.kv_host(), kv_ref, pos, B)
    print(f"  max|dlogit|/rms = {err:.2e}")
    m.close()


@pytest.mark.parametrize("accept", [2, 6])
def test_paged_verify_matches_oracle(torch_cuda, accept):
    """Verify (anchor + 7 drafts) on the small hybrid model with a paged cache
    whose 8 new rows straddle a page boundary."""
    from oracle import step as ostep
    from tests.harness import HostWeights, host_kv, kv_copy
    from tests.test_gpu_parity import _greedy_drafts, _gpu_verify
    w = paged(WL.mini_hybrid(), 32)
    n = 8
    p0 = 32 - 3
    W = HostWeights(w)
    kv = host_kv(w)
    toks = _greedy_drafts(w, W, kv, p0, accept, n)
    print(f"case {w.name} verify accept={accept} p0={p0}", flush=True)
    kv_ref = kv_copy(kv)
    v = ostep.verify_step(w, W, np.array([toks]), np.array([p0]), kv_ref)
    assert int(v["accept_len"][0]) == accept
    m = _model(w, shuffled_table(w, 11))
    logits, ids, acc, nxt = _gpu_verify(m, toks, p0)
    assert acc == accept
    err = GU.compare_verify(w, logits, ids, acc, nxt, v, f"paged verify a={accept}")
    kvg = m.kv_host()
    for j in range(n):
        GU.compare_kv_rows(w, kvg, kv_ref, [p0 + j], 1)
    print(f"  max|dlogit|/rms = {err:.2e}")
    m.close()


@pytest.mark.parametrize("name", ["mini_moe", "mini_hybrid"])
def test_fork_shares_prefix_pages(torch_cuda, name):
    """Sequence 1 forks sequence 0 at position p0: its block table points at
    sequence 0's full pages (shared, read only), its page holding p0 is a
    copy of sequence 0's (md_kv_copy_pages: copy-on-write) and its delta-rule
    states a copy of slot 0's (md_kv_copy_slot).  One step of both with the
    same token: bitwise equal logits, equal to the oracle's step of a batch
    whose slot 1 holds slot 0's history; each writes its new row into its
    own page and the shared pages stay as they were."""
    torch = torch_cuda
    from tests.harness import host_kv
    w = paged(WL.get(name), 32)
    P = w.kv_page
    bt = shuffled_table(w, 21)
    m = _model(w, bt)
    p0 = w.context
    j0 = p0 // P                      # the page that receives row p0
    fork = bt.copy()
    fork[1, :j0] = bt[0, :j0]         # shared prefix pages
    m.copy_pages([int(bt[0, j0])], [int(bt[1, j0])])   # sequence 1's own copy of the partial page
    m.copy_slot(0, 1)
    torch.cuda.synchronize(m.device)
    m.set_block_table(fork)
    before = [a.copy() for a in m.kv_host()]
    tok = int(synth.tokens(w, 1)[0])
    g = GU.run_gpu_step(m, [tok, tok], [p0, p0])
    assert np.array_equal(g["logits"][0], g["logits"][1]), "forked sequences differ"
    assert g["next"][0] == g["next"][1]
    kv = host_kv(w)
    for l in range(w.n_layers):
        kind = w.layer_kind(l)
        if kind == "gqa":
            kv[l][:, 1] = kv[l][:, 0]
        else:
            kv[l][1] = kv[l][0]
    o, kv_ref = GU.run_oracle_step(w, [tok, tok], [p0, p0], kv=kv)
    GU.compare_step(w, g, o, f"fork {name}")
    after = m.kv_host()
    GU.compare_kv_rows(w, after, kv_ref, [p0, p0], 2)
    # sequence 0's rows before p0 (including the shared pages) are untouched
    for l in range(w.n_layers):
        kind = w.layer_kind(l)
        if kind == "gqa":
            assert np.array_equal(after[l][:, 0, :, :p0], before[l][:, 0, :, :p0]), l
        elif kind == "mla":
            assert np.array_equal(after[l][0, :p0], before[l][0, :p0]), l
    m.close()


def test_copy_slot_contiguous(torch_cuda):
    """md_kv_copy_slot on a contiguous cache: slot 0's cache rows and
    delta-rule states become slot 3's, bit for bit; the others stay."""
    from decode_megakernel_md_amd.model import DeviceModel
    w = WL.mini_hybrid()
    m = DeviceModel(w)
    before = m.kv_host()
    m.copy_slot(0, 3)
    torch_cuda.cuda.synchronize(m.device)
    after = m.kv_host()
    for l in range(w.n_layers):
        a, b = after[l], before[l]
        if w.layer_kind(l) == "gqa":
            a, b = a.swapaxes(0, 1), b.swapaxes(0, 1)
        assert np.array_equal(a[3], b[0]), l
        for s in (0, 1, 2, 4):
            assert np.array_equal(a[s], b[s]), (l, s)
    m.close()


def test_bad_page_id_is_reported(torch_cuda):
    """A block-table entry outside the pool: the step reads page 0 in its
    place, the device reports the error (MD_EDEVICE, 'page id'), and after a
    valid table is restored the next step runs cleanly.  A paged model also
    refuses the contiguous entry point."""
    torch = torch_cuda
    from decode_megakernel_md_amd import _lib
    w = paged(WL.mini_dense(), 32)
    bt = shuffled_table(w, 5)
    m = _model(w, bt)
    dev = m.device
    t = torch.tensor(synth.tokens(w, 1), dtype=torch.int32, device=dev)
    p = torch.tensor([w.context], dtype=torch.int32, device=dev)
    logits = torch.empty((1, w.vocab), dtype=torch.float32, device=dev)
    L = _lib.lib()
    st = L.md_decode_step(m.handle, ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(p.data_ptr()),
                          ctypes.c_void_p(m.kv.data_ptr()), ctypes.c_void_p(logits.data_ptr()), 1, None, None,
                          ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == _lib.MD_EINVAL and "paged" in L.md_last_error().decode()
    bad = bt.copy()
    bad[0, 0] = w.kv_pages + 5
    m.set_block_table(bad)
    m.decode(t, p, logits)
    torch.cuda.synchronize(dev)
    with pytest.raises(_lib.MdError) as e:
        m.device_status()
    assert e.value.status == _lib.MD_EDEVICE and "page id" in str(e.value)
    m.set_block_table(bt)
    g = GU.run_gpu_step(m, list(synth.tokens(w, 1)), [w.context])
    o, _ = GU.run_oracle_step(w, list(synth.tokens(w, 1)), [w.context])
    GU.compare_step(w, g, o, "after a bad page id")
    m.close()
