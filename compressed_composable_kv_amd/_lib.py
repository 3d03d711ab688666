"""ctypes loader for libc2kv.so (the C2KV C ABI).

torch is imported first on purpose: its bundled HIP runtime then satisfies
libc2kv.so's libamdhip64.so.7 dependency, so the library and torch share one
runtime (and torch's streams are valid stream handles for the library).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading the library)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libc2kv.so")

c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_size_t = ctypes.c_size_t
c_float = ctypes.c_float
c_void_p = ctypes.c_void_p
c_char_p = ctypes.c_char_p
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_u64 = ctypes.POINTER(ctypes.c_uint64)
P_f32 = ctypes.POINTER(ctypes.c_float)


SEGMENT_HOST = 1   # C2KV_SEGMENT_HOST
SEGMENT_NO_REALIGN = 2   # C2KV_SEGMENT_NO_REALIGN
EXTRACT_ANCHOR = 1   # C2KV_EXTRACT_ANCHOR


class Segment(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("row_stride", c_int64),
                ("doc_len", c_int32), ("flags", c_int32)]


class TileEntry(ctypes.Structure):
    _fields_ = [("doc", c_int32), ("kv_head", c_int32), ("q_head", c_int32), ("q_slot", c_int32),
                ("q0", c_int32), ("q1", c_int32), ("k_slot", c_int32), ("key0", c_int32),
                ("nkeys", c_int32), ("masked", c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("attn_norm", c_void_p), ("wqkv", c_void_p), ("wqkv_c2", c_void_p), ("wo", c_void_p),
                ("ffn_norm", c_void_p), ("w_gate_up", c_void_p), ("w_down", c_void_p)]


# name -> (restype, argtypes)
SIGNATURES = {
    "c2kv_version": (c_char_p, []),
    "c2kv_status_string": (c_char_p, [c_int32]),
    "c2kv_last_error": (c_char_p, []),
    "c2kv_num_slots": (c_int32, [c_int32, c_int32]),
    "c2kv_slot_position": (c_int32, [c_int32, c_int32, c_int32]),
    "c2kv_rope_inv_freq": (c_int32, [c_int32, c_float, P_f32]),
    "c2kv_workspace_size_extract": (c_size_t, [P_i32, c_int32, c_int32, c_int32, c_int32, c_int32]),
    "c2kv_extract_attn": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    P_i32, c_int32, c_int32, c_int32,
                                    c_int32, c_int32, c_int32, c_float, c_int32,
                                    c_void_p, c_size_t, c_void_p]),
    "c2kv_extract_attn_ex": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       P_i32, c_int32, c_int32, c_int32,
                                       c_int32, c_int32, c_int32, c_float, c_int32, ctypes.c_uint32,
                                       c_void_p, c_size_t, c_void_p]),
    "c2kv_mask_cells_ex": (c_int32, [P_i32, c_int32, c_int32, c_int32, ctypes.c_uint32, P_u64, c_void_p, c_size_t,
                                     c_void_p]),
    "c2kv_workspace_size_extract_layer": (c_size_t, [P_i32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                                     c_int32, c_int32]),
    "c2kv_extract_layer": (c_int32, [c_void_p, c_void_p, ctypes.POINTER(LayerWeights), c_void_p, c_void_p,
                                     P_i32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                     c_int32, c_float, c_float, c_int32, c_void_p, c_size_t, c_void_p]),
    "c2kv_workspace_size_compose": (c_size_t, [c_int32]),
    "c2kv_compose": (c_int32, [ctypes.POINTER(Segment), c_int32, P_i32, c_int32, P_i32,
                               c_int32, c_int32, c_int32, c_float,
                               c_void_p, c_void_p, c_int64, c_void_p, P_i32, P_i32,
                               c_int32, c_void_p, c_size_t, c_void_p]),
    "c2kv_host_device_ptr": (c_int32, [c_void_p, c_size_t, ctypes.POINTER(c_void_p)]),
    "c2kv_workspace_size_compose_staged": (c_size_t, [ctypes.POINTER(Segment), c_int32, c_int32, c_int32, c_int32,
                                                      c_int32]),
    "c2kv_compose_staged": (c_int32, [ctypes.POINTER(Segment), c_int32, P_i32, c_int32, P_i32,
                                      c_int32, c_int32, c_int32, c_float,
                                      c_void_p, c_void_p, c_int64, c_void_p, P_i32, P_i32,
                                      c_int32, c_void_p, c_size_t, c_void_p]),
    "c2kv_workspace_size_prefill": (c_size_t, [P_i32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]),
    "c2kv_attn_prefill": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                    P_i32, P_i32, c_int32, c_int32, c_int32, c_int32, c_int32, c_float,
                                    c_void_p, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]),
    "c2kv_workspace_size_decode": (c_size_t, [P_i32, c_int32, c_int32, c_int32, c_int32, c_int32]),
    "c2kv_attn_decode": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                   P_i32, P_i32, c_int32, c_int32, c_int32, c_int32, c_float,
                                   c_void_p, c_void_p, c_int32, c_void_p, c_size_t, c_void_p]),
    "c2kv_attn_decode_noalloc": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                                           P_i32, P_i32, c_int32, c_int32, c_int32, c_int32, c_float,
                                           c_void_p, c_void_p, c_int32, c_void_p]),
    "c2kv_workspace_init": (c_int32, [c_void_p, c_size_t, c_void_p]),
    "c2kv_workspace_size_mask_cells": (c_size_t, []),
    "c2kv_mask_cells": (c_int32, [P_i32, c_int32, c_int32, c_int32, P_u64, c_void_p, c_size_t, c_void_p]),
    "c2kv_workspace_size_tile_schedule": (c_size_t, []),
    "c2kv_tile_schedule": (c_int32, [P_i32, c_int32, c_int32, c_int32, c_int32, c_int32, ctypes.c_uint32,
                                     c_void_p, c_int64, ctypes.POINTER(c_int64), c_void_p, c_size_t, c_void_p]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libc2kv.so; raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m compressed_composable_kv_amd.build_lib`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


STATUS = {0: "C2KV_OK", 1: "C2KV_ERR_INVALID_ARG", 2: "C2KV_ERR_UNSUPPORTED",
          3: "C2KV_ERR_WORKSPACE", 4: "C2KV_ERR_CAPACITY", 5: "C2KV_ERR_HIP"}


class C2KVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != 0:
        msg = load().c2kv_last_error().decode(errors="replace")
        raise C2KVError(status, msg)
