"""ctypes binding of the C ABI in include/mtpd.h (argument marshalling only).

Every compute step runs in the HIP library libmtpd.so next to this file. If that library is missing or cannot be
loaded, `lib()` raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmtpd.so")

MTPD_OK, MTPD_EINVAL, MTPD_ESHAPE, MTPD_ENOMEM, MTPD_EHIP, MTPD_EUNSUP = 0, -1, -2, -3, -4, -5
MTPD_MAX_BATCH = 256
MTPD_MAX_TIMED = 4096
SYMBOLS = ("mtpd_create", "mtpd_destroy", "mtpd_workspace_bytes", "mtpd_drafter_step", "mtpd_draft_block",
           "mtpd_masked_head", "mtpd_last_error", "mtpd_abi_version", "mtpd_timing_enable", "mtpd_timing_read",
           "mtpd_draft_block_sampled", "mtpd_sample_head", "mtpd_drafter_step_noalloc", "mtpd_set_option",
           "mtpd_fault_status", "mtpd_stream_read")
# handle options (include/mtpd.h)
MTPD_OPT_GRAPHS, MTPD_OPT_PERSISTENT, MTPD_OPT_DENSE_PATH, MTPD_OPT_ATTN_VALU = 1, 2, 3, 4
MTPD_NOALLOC_SCRATCH_BYTES = 8 << 20

u16p = C.POINTER(C.c_uint16)
i32p = C.POINTER(C.c_int32)
f32p = C.POINTER(C.c_float)


class mtpd_config(C.Structure):
    _fields_ = [("backbone", C.c_int32), ("hidden", C.c_int32), ("n_layer", C.c_int32), ("n_head", C.c_int32),
                ("n_kv_head", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("n_centroids", C.c_int32), ("top_k", C.c_int32), ("swa_window", C.c_int32),
                ("full_attn_layers", C.c_uint32), ("rms_eps", C.c_float), ("attn_scale", C.c_float),
                ("embed_scale", C.c_float)]


class mtpd_layer(C.Structure):
    _fields_ = [("attn_q", C.c_void_p), ("attn_q_norm", C.c_void_p), ("attn_output", C.c_void_p),
                ("attn_norm", C.c_void_p), ("post_attention_norm", C.c_void_p), ("ffn_norm", C.c_void_p),
                ("post_ffw_norm", C.c_void_p), ("ffn_gate", C.c_void_p), ("ffn_up", C.c_void_p),
                ("ffn_down", C.c_void_p), ("layer_output_scale", C.c_float)]


class mtpd_weights(C.Structure):
    _fields_ = [("pre_proj", C.c_void_p), ("post_proj", C.c_void_p), ("output_norm", C.c_void_p),
                ("token_embd", C.c_void_p), ("centroids", C.c_void_p), ("token_ordering", C.c_void_p),
                ("layers", C.POINTER(mtpd_layer))]


class mtpd_kv(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("cap", C.c_int32), ("shared", C.c_int32), ("len", i32p),
                ("first", i32p)]


class mtpd_shared_kv(C.Structure):
    _fields_ = [("sliding", mtpd_kv), ("full", mtpd_kv), ("rope", C.c_void_p)]


_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """Load libmtpd.so (built in-tree by mtp_drafter_step_amd.build); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing (run mtp_drafter_step_amd/build.py)")
    L = C.CDLL(LIB_PATH)
    vp, sz = C.c_void_p, C.c_size_t
    L.mtpd_create.argtypes = [C.POINTER(mtpd_config), C.POINTER(mtpd_weights), C.c_int32, C.POINTER(vp)]
    L.mtpd_create.restype = C.c_int
    L.mtpd_destroy.argtypes = [vp]
    L.mtpd_destroy.restype = None
    L.mtpd_workspace_bytes.argtypes = [vp, C.c_int32]
    L.mtpd_workspace_bytes.restype = sz
    L.mtpd_drafter_step.argtypes = [vp, vp, vp, C.c_int32, vp, vp, vp, C.POINTER(mtpd_shared_kv), vp, vp, vp, vp, vp,
                                    vp]
    L.mtpd_drafter_step.restype = C.c_int
    L.mtpd_drafter_step_noalloc.argtypes = [vp, vp, C.c_int32, vp, vp, vp, C.POINTER(mtpd_shared_kv), vp, vp, vp, vp,
                                            vp, vp]
    L.mtpd_drafter_step_noalloc.restype = C.c_int
    L.mtpd_draft_block.argtypes = [vp, vp, vp, C.c_int32, C.c_int32, vp, vp, vp, C.POINTER(mtpd_shared_kv), vp, vp,
                                   vp]
    L.mtpd_draft_block.restype = C.c_int
    L.mtpd_masked_head.argtypes = [vp, vp, vp, C.c_int32, vp, vp, vp, vp, vp, vp]
    L.mtpd_masked_head.restype = C.c_int
    L.mtpd_draft_block_sampled.argtypes = [vp, vp, vp, C.c_int32, C.c_int32, vp, vp, vp, vp, C.c_float, vp, vp, vp,
                                           vp, vp]
    L.mtpd_draft_block_sampled.restype = C.c_int
    L.mtpd_sample_head.argtypes = [vp, vp, vp, C.c_int32, vp, C.c_float, vp, vp, vp, vp]
    L.mtpd_sample_head.restype = C.c_int
    L.mtpd_last_error.argtypes = []
    L.mtpd_last_error.restype = C.c_char_p
    L.mtpd_abi_version.argtypes = []
    L.mtpd_abi_version.restype = C.c_int32
    L.mtpd_set_option.argtypes = [vp, C.c_int32, C.c_int32]
    L.mtpd_set_option.restype = C.c_int
    L.mtpd_fault_status.argtypes = [vp, C.c_int32]
    L.mtpd_fault_status.restype = C.c_int32
    L.mtpd_stream_read.argtypes = [vp, C.c_uint64, C.c_uint32, vp, vp]
    L.mtpd_stream_read.restype = C.c_int
    L.mtpd_timing_enable.argtypes = [vp, C.c_int32]
    L.mtpd_timing_enable.restype = C.c_int
    L.mtpd_timing_read.argtypes = [vp, C.c_int32, C.POINTER(C.c_char_p), f32p]
    L.mtpd_timing_read.restype = C.c_int32
    _lib = L
    return L


class MtpdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mtpd error {code}: {msg}")
        self.code = code


def check(rc: int) -> None:
    if rc != MTPD_OK:
        raise MtpdError(rc, lib().mtpd_last_error().decode())
