"""Device-side model: weights, workspace and KV / state buffers in HBM
(allocated through PyTorch), handed to libmd.so.

Inputs come from the seeded `synth` generator, drawn straight into device
memory.  Nothing here computes any part of the decode step."""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import numpy as np

import synth
from synth.workloads import V_TILE, Workload, kv_layout, kv_pool_layout, tensor_inventory

from . import _lib
from ._lib import check, config_from, lib


def v_logical(v: np.ndarray) -> np.ndarray:
    """A GQA V cache [.., max_ctx, head_dim] as stored (V_TILE-position tiles,
    dim-major within a tile) -> the same values in row order."""
    *lead, C, D = v.shape
    t = v.reshape(*lead, C // V_TILE, D, V_TILE)
    return np.swapaxes(t, -1, -2).reshape(*lead, C, D)


def _align(x: int, a: int = 256) -> int:
    return (x + a - 1) // a * a


class DeviceModel:
    """One model instance on one GPU.

    overrides: optional {tensor name: uint16 host array} replacing drawn
    weights (used by tests that pin special cases).

    Paged caches (w.kv_page > 0): self.kv is the page pool and self.bt the
    block table (int32 [max_batch][max_ctx / kv_page], device); block_table
    gives its initial contents (default: slot s, page j -> s * (max_ctx /
    kv_page) + j).  The seeded synthetic cache of every slot is drawn in the
    contiguous layout and scattered into the pages the table names; pages
    no slot maps are filled with NaN, so that a read of a wrong page shows."""

    def __init__(self, w: Workload, device: str = "cuda:0", overrides: Optional[Dict[str, np.ndarray]] = None,
                 block_table: Optional[np.ndarray] = None):
        import torch

        self.torch = torch
        self.w = w
        self.device = torch.device(device)
        self.cfg = config_from(w)
        L = lib()
        inv = _lib.weight_inventory(self.cfg)
        specs = tensor_inventory(w)
        if [(s.name, s.rows, s.cols) for s in specs] != inv:
            raise RuntimeError("library weight inventory differs from the workload's tensor list")
        self.specs = specs
        # matrices are stored tiled (md_pack_weight), norm gains as plain vectors
        self.packed = [L.md_weight_layout(ctypes.byref(self.cfg), i) == 1 for i in range(len(specs))]
        self.sizes = [L.md_packed_bytes(s.rows, s.cols) if pk else s.numel * 2 for s, pk in zip(specs, self.packed)]
        self.offsets = []
        off = 0
        for n in self.sizes:
            self.offsets.append(off)
            off = _align(off + n)
        self.weight_bytes = sum(s.numel * 2 for s in specs)
        stream = torch.cuda.current_stream(self.device)
        sptr = stream.cuda_stream
        self.wbuf = torch.empty(off, dtype=torch.uint8, device=self.device)
        base = self.wbuf.data_ptr()
        overrides = overrides or {}
        stage = torch.empty(max(s.numel * 2 for s in specs), dtype=torch.uint8, device=self.device)
        for s, o, pk in zip(specs, self.offsets, self.packed):
            dst = stage if pk else self.wbuf[o:o + s.numel * 2]
            if s.name in overrides:
                a = np.ascontiguousarray(overrides[s.name], dtype=np.uint16).reshape(-1)
                assert a.size == s.numel
                dst[:s.numel * 2].copy_(torch.from_numpy(a.view(np.uint8)))
            elif s.kind == "gain" and s.sigma != 0.0:
                a = synth.weight_host(w, s).reshape(-1)
                dst[:s.numel * 2].copy_(torch.from_numpy(a.view(np.uint8)))
            else:
                synth.weight_device(w, s, dst.data_ptr(), sptr)
            if pk:
                check(L.md_pack_weight(ctypes.c_void_p(stage.data_ptr()), ctypes.c_void_p(base + o), s.rows, s.cols,
                                       ctypes.c_void_p(sptr)))
        torch.cuda.synchronize(self.device)
        del stage
        self.ws_bytes = L.md_workspace_bytes(ctypes.byref(self.cfg))
        if self.ws_bytes == 0:  # the configuration was rejected: surface the library's reason
            check(L.md_init_model(ctypes.byref(self.cfg), None, 0, None, 0, None, ctypes.byref(ctypes.c_void_p())))
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.kv_bytes = L.md_kv_bytes(ctypes.byref(self.cfg), self.cfg.max_batch, self.cfg.max_ctx)
        self.paged = w.kv_page > 0
        lay, total = kv_pool_layout(w) if self.paged else kv_layout(w)
        if total != self.kv_bytes:
            raise RuntimeError(f"KV layout mismatch: library {self.kv_bytes} vs workload {total}")
        self.kv_layout = lay
        self.kv = torch.empty(self.kv_bytes, dtype=torch.uint8, device=self.device)
        self.bt = None
        if self.paged:
            npp = w.max_ctx // w.kv_page
            if block_table is None:
                block_table = np.arange(w.max_batch * npp, dtype=np.int32).reshape(w.max_batch, npp)
            self.set_block_table(block_table)
        self.reset_kv()
        ptrs = (ctypes.c_void_p * len(specs))(*[base + o for o in self.offsets])
        h = ctypes.c_void_p()
        torch.cuda.synchronize(self.device)
        check(L.md_init_model(ctypes.byref(self.cfg), ptrs, len(specs), ctypes.c_void_p(self.ws.data_ptr()),
                              self.ws_bytes, ctypes.c_void_p(sptr), ctypes.byref(h)))
        self.handle = h

    # ------------------------------------------------------------------ state
    def set_block_table(self, bt: np.ndarray) -> None:
        """Block table of a paged model (host int32 [max_batch][max_ctx / kv_page]), copied to the device."""
        w = self.w
        bt = np.ascontiguousarray(bt, dtype=np.int32)
        assert bt.shape == (w.max_batch, w.max_ctx // w.kv_page), bt.shape
        self.bt_host = bt
        self.bt = self.torch.from_numpy(bt).to(self.device)

    def reset_kv(self) -> None:
        """Redraw every layer's cache / state from the seeded generator (paged:
        each slot's contiguous draw scattered into the pages of the block table)."""
        torch = self.torch
        sptr = torch.cuda.current_stream(self.device).cuda_stream
        base = self.kv.data_ptr()
        if not self.paged:
            for l, (kind, off, nbytes, shape, dt) in enumerate(self.kv_layout):
                synth.kv_layer_device(self.w, l, base + off, sptr)
            return
        w = self.w
        clay, _ = kv_layout(w)
        P, N, Bm, C = w.kv_page, w.kv_pages, w.max_batch, w.max_ctx
        idx = torch.from_numpy(self.bt_host.reshape(-1).astype(np.int64)).to(self.device)
        for l, (kind, off, nbytes, shape, dt) in enumerate(self.kv_layout):
            if kind == "kda":
                synth.kv_layer_device(w, l, base + off, sptr)
                continue
            tmp = torch.empty(clay[l][2], dtype=torch.uint8, device=self.device)
            synth.kv_layer_device(w, l, tmp.data_ptr(), sptr)
            pool = self.kv[off:off + nbytes].view(torch.int16)
            pool.fill_(0x7FC0)  # NaN: pages no slot maps
            src = tmp.view(torch.int16)
            if kind == "gqa":
                nkv, hd = w.n_kv_heads, w.head_dim
                half = Bm * nkv * C * hd
                k = src[:half].view(Bm, nkv, C // P, P, hd).permute(0, 2, 1, 3, 4).reshape(Bm * (C // P), nkv, P, hd)
                v = src[half:].view(Bm, nkv, C // P, P // V_TILE, hd, V_TILE).permute(0, 2, 1, 3, 4, 5)
                v = v.reshape(Bm * (C // P), nkv, P // V_TILE, hd, V_TILE)
                pk = pool[:N * nkv * P * hd].view(N, nkv, P, hd)
                pv = pool[N * nkv * P * hd:].view(N, nkv, P // V_TILE, hd, V_TILE)
                pk[idx] = k
                pv[idx] = v
            else:
                rows = src.view(Bm, C // P, P, w.mla_row).reshape(Bm * (C // P), P, w.mla_row)
                pool.view(N, P, w.mla_row)[idx] = rows
            del tmp
        torch.cuda.synchronize(self.device)

    def kv_layer(self, l: int):
        """Device tensor view of layer l's cache / state as stored (shape per
        synth.kv_layout; for a GQA layer, index 1 is V in its stored tile
        order: view it with v_logical)."""
        torch = self.torch
        kind, off, nbytes, shape, dt = self.kv_layout[l]
        raw = self.kv[off:off + nbytes]
        if kind == "kda":
            return raw.view(torch.float32).view(*shape)
        if kind == "gqa":
            return raw.view(torch.int16).view(2, *shape)
        return raw.view(torch.int16).view(*shape)

    def kv_host(self):
        """Host copies of every layer's cache / state in the oracle's layout
        (GQA V converted from its tiles to [max_batch][n_kv][max_ctx][head_dim];
        a paged model's pages gathered through its block table)."""
        if self.paged:
            return self._kv_host_paged()
        out = []
        for l in range(self.w.n_layers):
            t = self.kv_layer(l).cpu().numpy()
            if t.dtype == np.int16:
                t = t.view(np.uint16)
            if self.kv_layout[l][0] == "gqa":
                t = np.stack([t[0], v_logical(t[1])])
            out.append(np.ascontiguousarray(t))
        return out

    def _kv_host_paged(self):
        w = self.w
        P, N, Bm, C = w.kv_page, w.kv_pages, w.max_batch, w.max_ctx
        bt = self.bt_host.reshape(-1)
        out = []
        for l, (kind, off, nbytes, shape, dt) in enumerate(self.kv_layout):
            raw = self.kv[off:off + nbytes].cpu().numpy()
            if kind == "kda":
                out.append(np.ascontiguousarray(raw.view(np.float32).reshape(shape)))
                continue
            a = raw.view(np.uint16)
            if kind == "gqa":
                nkv, hd = w.n_kv_heads, w.head_dim
                pk = a[:N * nkv * P * hd].reshape(N, nkv, P, hd)[bt].reshape(Bm, C // P, nkv, P, hd)
                pv = a[N * nkv * P * hd:].reshape(N, nkv, P // V_TILE, hd, V_TILE)[bt]
                pv = pv.reshape(Bm, C // P, nkv, P // V_TILE, hd, V_TILE)
                k = pk.transpose(0, 2, 1, 3, 4).reshape(Bm, nkv, C, hd)
                vt = pv.transpose(0, 2, 1, 3, 4, 5).reshape(Bm, nkv, C // V_TILE, hd, V_TILE)
                v = np.swapaxes(vt, -1, -2).reshape(Bm, nkv, C, hd)
                out.append(np.ascontiguousarray(np.stack([k, v])))
            else:
                rows = a.reshape(N, P, w.mla_row)[bt].reshape(Bm, C, w.mla_row)
                out.append(np.ascontiguousarray(rows))
        return out

    # ------------------------------------------------------------------ steps
    def decode(self, tokens, positions, logits, out_tokens=None, out_ids=None, multilaunch=False, stream=None,
               noalloc=False):
        """Enqueue one decode step.  All tensors are device tensors.
        multilaunch: one launch per phase; noalloc: the allocation-free step
        (scratch from the library's static array)."""
        torch = self.torch
        B = int(tokens.shape[0])
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        if self.paged:
            if multilaunch or noalloc:
                raise ValueError("a paged model runs the megakernel step (md_decode_step_paged) only")
            check(lib().md_decode_step_paged(self.handle, ctypes.c_void_p(tokens.data_ptr()),
                                             ctypes.c_void_p(positions.data_ptr()), ctypes.c_void_p(self.kv.data_ptr()),
                                             ctypes.c_void_p(self.bt.data_ptr()), ctypes.c_void_p(logits.data_ptr()), B,
                                             ctypes.c_void_p(out_tokens.data_ptr() if out_tokens is not None else 0),
                                             ctypes.c_void_p(out_ids.data_ptr() if out_ids is not None else 0),
                                             ctypes.c_void_p(s.cuda_stream)))
            return
        fn = (lib().md_decode_step_multilaunch if multilaunch else
              lib().md_decode_step_noalloc if noalloc else lib().md_decode_step)
        check(fn(self.handle, ctypes.c_void_p(tokens.data_ptr()), ctypes.c_void_p(positions.data_ptr()),
                 ctypes.c_void_p(self.kv.data_ptr()), ctypes.c_void_p(logits.data_ptr()), B,
                 ctypes.c_void_p(out_tokens.data_ptr() if out_tokens is not None else 0),
                 ctypes.c_void_p(out_ids.data_ptr() if out_ids is not None else 0),
                 ctypes.c_void_p(s.cuda_stream)))

    def verify(self, tokens, positions, logits, accept_len, next_token, out_ids=None, stream=None):
        """Enqueue one verify of tokens[1, n] (anchor + drafts) at positions[1]."""
        torch = self.torch
        B, n = int(tokens.shape[0]), int(tokens.shape[1])
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        if self.paged:
            check(lib().md_verify_step_paged(self.handle, ctypes.c_void_p(tokens.data_ptr()),
                                             ctypes.c_void_p(positions.data_ptr()), ctypes.c_void_p(self.kv.data_ptr()),
                                             ctypes.c_void_p(self.bt.data_ptr()), ctypes.c_void_p(logits.data_ptr()),
                                             ctypes.c_void_p(accept_len.data_ptr()),
                                             ctypes.c_void_p(next_token.data_ptr()),
                                             ctypes.c_void_p(out_ids.data_ptr() if out_ids is not None else 0), B, n,
                                             ctypes.c_void_p(s.cuda_stream)))
            return
        check(lib().md_verify_step(self.handle, ctypes.c_void_p(tokens.data_ptr()),
                                   ctypes.c_void_p(positions.data_ptr()), ctypes.c_void_p(self.kv.data_ptr()),
                                   ctypes.c_void_p(logits.data_ptr()), ctypes.c_void_p(accept_len.data_ptr()),
                                   ctypes.c_void_p(next_token.data_ptr()),
                                   ctypes.c_void_p(out_ids.data_ptr() if out_ids is not None else 0), B, n,
                                   ctypes.c_void_p(s.cuda_stream)))

    def copy_pages(self, src, dst, stream=None) -> None:
        """md_kv_copy_pages: page src[i] -> dst[i] of every GQA / MLA layer (int sequences)."""
        torch = self.torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        a = torch.tensor(list(src), dtype=torch.int32, device=self.device)
        b = torch.tensor(list(dst), dtype=torch.int32, device=self.device)
        check(lib().md_kv_copy_pages(self.handle, ctypes.c_void_p(self.kv.data_ptr()), ctypes.c_void_p(a.data_ptr()),
                                     ctypes.c_void_p(b.data_ptr()), len(a), ctypes.c_void_p(s.cuda_stream)))
        torch.cuda.synchronize(self.device)

    def copy_slot(self, src: int, dst: int, stream=None) -> None:
        """md_kv_copy_slot: sequence slot src -> dst (delta-rule states; contiguous caches' rows too)."""
        torch = self.torch
        s = stream if stream is not None else torch.cuda.current_stream(self.device)
        check(lib().md_kv_copy_slot(self.handle, ctypes.c_void_p(self.kv.data_ptr()), src, dst,
                                    ctypes.c_void_p(s.cuda_stream)))

    def device_status(self) -> None:
        check(lib().md_get_device_status(self.handle))

    def close(self) -> None:
        """Free the library handle and every device buffer of the model (after
        the device has finished with them), so that nothing of it is left for
        the runtime's own teardown at interpreter exit."""
        if getattr(self, "handle", None):
            self.torch.cuda.synchronize(self.device)
            lib().md_free_model(self.handle)
            self.handle = None
        for name in ("wbuf", "ws", "kv", "bt"):
            if getattr(self, name, None) is not None:
                setattr(self, name, None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
