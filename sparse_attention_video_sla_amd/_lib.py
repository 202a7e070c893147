"""ctypes loader for libsla.so, the gfx950 HIP library behind include/sla.h.

There is no fallback: if the library is missing or cannot be loaded, every
entry point raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsla.so")

SLA_OK, SLA_ERR_INVALID_ARG, SLA_ERR_UNSUPPORTED, SLA_ERR_WORKSPACE, SLA_ERR_DEVICE = range(5)
SLA_F32, SLA_BF16 = 0, 1
SLA_PHI_SOFTMAX = 0
NOALLOC_SCRATCH_BYTES = 512 << 20   # SLA_NOALLOC_SCRATCH_BYTES

# every symbol include/sla.h declares
EXPORTS = ("sla_version", "sla_counts", "sla_workspace_size", "sla_pool", "sla_classify",
           "sla_forward", "sla_forward_noalloc", "sla_forward_save", "sla_backward_saved", "sla_lists_workspace_size", "sla_forward_lists", "sla_lvsa_plan", "sla_lvsa_sets",
           "sla_lvsa_workspace_size", "sla_forward_lvsa", "sla_sta_tile_order",
           "sla_sta_workspace_size", "sla_forward_sta", "sla_backward_workspace_size",
           "sla_backward", "sla_block_mass", "sla_mask_stats", "sla_set_stage_timing", "sla_stage_times",
           "sla_last_error")
STAGES = ("pool", "classify", "state", "assemble", "fused")

_lib = None


class SlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("sla status %d: %s" % (status, message))
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libsla.so not found at %s: build it with "
                           "`python -m sparse_attention_video_sla_amd.build`" % path)
    L = ctypes.CDLL(path)
    P, I, D, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_size_t
    L.sla_version.restype = I
    L.sla_version.argtypes = []
    L.sla_last_error.restype = ctypes.c_char_p
    L.sla_last_error.argtypes = []
    L.sla_counts.restype = I
    L.sla_counts.argtypes = [I, D, D, ctypes.POINTER(I), ctypes.POINTER(I)]
    L.sla_workspace_size.restype = I
    L.sla_workspace_size.argtypes = [I, I, I, I, I, I, D, D, ctypes.POINTER(SZ)]
    L.sla_pool.restype = I
    L.sla_pool.argtypes = [P, P, I, I, I, I, I, I, P, P, P]
    L.sla_classify.restype = I
    L.sla_classify.argtypes = [P, P, I, I, I, I, D, D, P, P, P, P, P]
    L.sla_forward.restype = I
    L.sla_forward.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, D, I, P, P, P, SZ, P]
    L.sla_forward_noalloc.restype = I
    L.sla_forward_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, D, I, P, P, P]
    L.sla_lists_workspace_size.restype = I
    L.sla_lists_workspace_size.argtypes = [I, I, I, I, ctypes.POINTER(SZ)]
    L.sla_forward_lists.restype = I
    L.sla_forward_lists.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, I, P, P, SZ, P]
    IP = ctypes.POINTER(ctypes.c_int)
    L.sla_lvsa_plan.restype = I
    L.sla_lvsa_plan.argtypes = [I, I, I, IP, IP, IP]
    L.sla_lvsa_sets.restype = I
    L.sla_lvsa_sets.argtypes = [I, I, I, I, P, P, I, P]
    L.sla_lvsa_workspace_size.restype = I
    L.sla_lvsa_workspace_size.argtypes = [I, I, I, I, I, I, ctypes.POINTER(SZ)]
    L.sla_forward_lvsa.restype = I
    L.sla_forward_lvsa.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I, I, I, P, P, SZ, P]
    L.sla_sta_tile_order.restype = I
    L.sla_sta_tile_order.argtypes = [I, I, I, I, I, I, P]
    L.sla_sta_workspace_size.restype = I
    L.sla_sta_workspace_size.argtypes = [I] * 11 + [ctypes.POINTER(SZ)]
    L.sla_forward_sta.restype = I
    L.sla_forward_sta.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I, I, I, I, I, I, I, P, P, SZ, P]
    D_ = ctypes.c_double
    L.sla_backward_workspace_size.restype = I
    L.sla_backward_workspace_size.argtypes = [I, I, I, I, I, D_, D_, ctypes.POINTER(SZ)]
    L.sla_backward.restype = I
    L.sla_backward.argtypes = [P, P, P, P, P, I, I, I, I, I, I, D_, D_, I, P, P, P, P, P, SZ, P]
    L.sla_forward_save.restype = I
    L.sla_forward_save.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D_, D_, I, P, P, P, SZ, P]
    L.sla_backward_saved.restype = I
    L.sla_backward_saved.argtypes = [P, P, P, P, P, I, I, I, I, I, I, D_, D_, I, P, P, P, P, P, SZ, P]
    L.sla_block_mass.restype = I
    L.sla_block_mass.argtypes = [P, P, I, I, I, I, I, I, P, P]
    L.sla_mask_stats.restype = I
    L.sla_mask_stats.argtypes = [P, P, ctypes.c_long, I, P, P]
    L.sla_set_stage_timing.restype = I
    L.sla_set_stage_timing.argtypes = [I]
    L.sla_stage_times.restype = I
    L.sla_stage_times.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(I)]
    _lib = L
    return L


def check(status: int) -> None:
    if status != SLA_OK:
        raise SlaError(status, load().sla_last_error().decode(errors="replace"))
