"""ctypes binding of include/md.h: argument marshalling only.

Every step of the decode path runs in libmd.so's HIP kernels; this module
never computes anything and raises if the library is missing."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "libmd.so")

MD_OK, MD_EINVAL, MD_EUNSUPPORTED, MD_ENOMEM, MD_EHIP, MD_EDEVICE = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "MD_OK", -1: "MD_EINVAL", -2: "MD_EUNSUPPORTED", -3: "MD_ENOMEM", -4: "MD_EHIP", -5: "MD_EDEVICE"}

I32 = ctypes.c_int32


class MdConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", I32), ("hidden", I32), ("vocab", I32), ("max_batch", I32), ("max_ctx", I32),
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("attn_kind", I32),
        ("n_q_heads", I32), ("n_kv_heads", I32), ("head_dim", I32),
        ("mla_every", I32), ("mla_heads", I32), ("q_lora", I32), ("kv_lora", I32), ("rope_dim", I32),
        ("nope_dim", I32), ("v_dim", I32),
        ("kda_heads", I32), ("kda_dk", I32), ("kda_dv", I32), ("kda_qk_l2norm", I32),
        ("ffn_dim", I32),
        ("n_experts", I32), ("top_k", I32), ("expert_ffn", I32), ("n_shared", I32), ("shared_ffn", I32),
        ("norm_topk", I32),
        ("flags", I32),
        ("kv_page", I32), ("kv_pages", I32),
    ]


class MdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


EXPORTS = [
    "md_weight_count", "md_weight_info", "md_workspace_bytes", "md_kv_bytes", "md_init_model",
    "md_decode_step", "md_decode_step_multilaunch", "md_decode_step_noalloc", "md_verify_step", "md_get_device_status",
    "md_last_error", "md_free_model", "md_set_trace", "md_grid_size", "md_packed_bytes", "md_pack_weight",
    "md_weight_layout", "md_decode_step_paged", "md_verify_step_paged", "md_kv_copy_pages", "md_kv_copy_slot",
]

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            raise RuntimeError(f"{SO} is not built; run __graft_entry__.build() (no fallback exists)")
        L = ctypes.CDLL(SO)
        P = ctypes.c_void_p
        CFG = ctypes.POINTER(MdConfig)
        L.md_weight_count.restype = ctypes.c_size_t
        L.md_weight_count.argtypes = [CFG]
        L.md_weight_info.restype = I32
        L.md_weight_info.argtypes = [CFG, ctypes.c_size_t, ctypes.c_char_p, ctypes.c_size_t,
                                     ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        L.md_workspace_bytes.restype = ctypes.c_size_t
        L.md_workspace_bytes.argtypes = [CFG]
        L.md_kv_bytes.restype = ctypes.c_size_t
        L.md_kv_bytes.argtypes = [CFG, I32, I32]
        L.md_init_model.restype = I32
        L.md_init_model.argtypes = [CFG, ctypes.POINTER(P), ctypes.c_size_t, P, ctypes.c_size_t, P, ctypes.POINTER(P)]
        for fn in ("md_decode_step", "md_decode_step_multilaunch", "md_decode_step_noalloc"):
            f = getattr(L, fn)
            f.restype = I32
            f.argtypes = [P, P, P, P, P, I32, P, P, P]
        L.md_verify_step.restype = I32
        L.md_verify_step.argtypes = [P, P, P, P, P, P, P, P, I32, I32, P]
        L.md_get_device_status.restype = I32
        L.md_get_device_status.argtypes = [P]
        L.md_last_error.restype = ctypes.c_char_p
        L.md_last_error.argtypes = []
        L.md_set_trace.restype = I32
        L.md_set_trace.argtypes = [P, P, I32]
        L.md_grid_size.restype = I32
        L.md_grid_size.argtypes = [P]
        L.md_weight_layout.restype = I32
        L.md_weight_layout.argtypes = [CFG, ctypes.c_size_t]
        L.md_packed_bytes.restype = ctypes.c_size_t
        L.md_packed_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.md_pack_weight.restype = I32
        L.md_pack_weight.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, P]
        L.md_decode_step_paged.restype = I32
        L.md_decode_step_paged.argtypes = [P, P, P, P, P, P, I32, P, P, P]
        L.md_verify_step_paged.restype = I32
        L.md_verify_step_paged.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, P]
        L.md_kv_copy_pages.restype = I32
        L.md_kv_copy_pages.argtypes = [P, P, P, P, I32, P]
        L.md_kv_copy_slot.restype = I32
        L.md_kv_copy_slot.argtypes = [P, P, I32, I32, P]
        L.md_free_model.restype = None
        L.md_free_model.argtypes = [P]
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != MD_OK:
        raise MdError(status, lib().md_last_error().decode())


def config_from(w) -> MdConfig:
    """md_config for a synth.workloads.Workload (field-for-field)."""
    c = MdConfig()
    for name, _ in MdConfig._fields_:
        if name == "flags":
            c.flags = 0
        else:
            setattr(c, name, getattr(w, name))
    return c


def weight_inventory(cfg: MdConfig):
    L = lib()
    n = L.md_weight_count(ctypes.byref(cfg))
    out = []
    buf = ctypes.create_string_buffer(128)
    r, k = ctypes.c_int64(), ctypes.c_int64()
    for i in range(n):
        check(L.md_weight_info(ctypes.byref(cfg), i, buf, 128, ctypes.byref(r), ctypes.byref(k)))
        out.append((buf.value.decode(), r.value, k.value))
    return out
