"""ctypes binding of libdg (include/dg.h, include/dg_test.h): argument marshalling only.

The library must have been built (``__graft_entry__.build()`` or
``python -m block_discrete_diffusion_dg_amd.build``); a missing library is an
error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

# The in-tree build; DG_LIB_PATH names another build of the same library
# (the host-side sanitizer build of the ABI tests).
LIB_PATH = os.environ.get("DG_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdg.so")

DG_OK, DG_EINVAL, DG_ECAPACITY, DG_EHIP, DG_ESTATE = 0, -1, -2, -3, -4
STATUS_NAMES = {0: "DG_OK", -1: "DG_EINVAL", -2: "DG_ECAPACITY", -3: "DG_EHIP", -4: "DG_ESTATE"}

c_i32 = ctypes.c_int32
c_f32 = ctypes.c_float
c_vp = ctypes.c_void_p
c_size = ctypes.c_size_t


class DGConfig(ctypes.Structure):
    _fields_ = [(n, c_i32) for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim",
                                     "n_experts", "top_k", "d_expert", "d_shared", "vocab",
                                     "canvas", "max_ctx", "max_requests", "max_rows")] + \
               [(n, c_f32) for n in ("rms_eps", "rope_theta", "tau_first", "tau_last")] + \
               [("expert_format", c_i32), ("d_selfcond", c_i32), ("lmhead_format", c_i32)]


WEIGHT_FORMAT = {"bf16": 0, "fp8": 1}


LAYER_FIELDS = ("attn_norm", "w_qkv", "w_o", "moe_norm", "w_router", "w_gate", "w_up", "w_down",
                "ws_gate", "ws_up", "ws_down")
# Streamed projection matrices: passed to dg_create in the fragment-major
# layout made by dg_pack_weight; the other fields stay row-major.
PACKED_FIELDS = ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")


# Expert matrices (bf16 fragment-major, or FP8 codes with row scales) and the
# fields holding their FP8 row scales, in the same order.
EXPERT_FIELDS = ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
SCALE_FIELDS = ("s_gate", "s_up", "s_down", "ss_gate", "ss_up", "ss_down")


class DGLayerWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in LAYER_FIELDS + SCALE_FIELDS]


class DGWeights(ctypes.Structure):
    _fields_ = [("embed", c_vp), ("final_norm", c_vp), ("layers", ctypes.POINTER(DGLayerWeights)),
                ("sc_gate", c_vp), ("sc_up", c_vp), ("sc_down", c_vp), ("embed_t", c_vp),
                ("embed_fp8", c_vp), ("embed_scale", c_vp)]


class DGRowStats(ctypes.Structure):
    _fields_ = [("max_logit", c_f32), ("log_z", c_f32), ("held_logit", c_f32), ("conf", c_f32),
                ("argmax", c_i32), ("accepted", c_i32), ("entropy", c_f32), ("sample", c_i32),
                ("sample_logit", c_f32), ("pad", c_i32)]


ROW_STATS_BYTES = ctypes.sizeof(DGRowStats)


class DGStepArgs(ctypes.Structure):
    _fields_ = [("n_req", c_i32), ("req", ctypes.POINTER(c_i32)), ("d_canvas", c_vp),
                ("d_committed", c_vp), ("step", c_i32), ("n_steps", c_i32),
                ("seed", ctypes.POINTER(ctypes.c_uint64)), ("block", ctypes.POINTER(c_i32)),
                ("d_stats", c_vp), ("confidence", c_i32), ("stop_entropy", c_f32), ("d_stop", c_vp),
                ("candidate", c_i32)]


CONFIDENCE = {"prob": 0, "entropy": 1}
CANDIDATE = {"argmax": 0, "sample": 1}


WS_FIELDS = ("h", "u", "q", "attn_o", "attn_part", "attn_ml", "rope", "z", "idx", "w", "wslot",
             "cnt", "off", "items", "perm", "slot", "hid", "hid_s", "y", "lm_part", "lm_gpart", "stats", "ids", "ss", "zpart", "sync",
             "prev", "sc_p", "sc_qpart", "sc_part", "sc_e", "sc_g", "sc_u", "sc_hid", "sc_out", "sc_state", "total")


class DGWsLayout(ctypes.Structure):
    _fields_ = [(n, c_size) for n in WS_FIELDS]


# name -> (restype, argtypes); every symbol declared in include/dg.h and include/dg_test.h
SIGNATURES = {
    "dg_kv_cache_bytes": (c_size, [ctypes.POINTER(DGConfig)]),
    "dg_workspace_bytes": (c_size, [ctypes.POINTER(DGConfig)]),
    "dg_create": (c_i32, [ctypes.POINTER(DGConfig), ctypes.POINTER(DGWeights), c_vp, c_vp, c_size,
                          ctypes.POINTER(c_vp)]),
    "dg_destroy": (None, [c_vp]),
    "dg_pack_weight": (c_i32, [c_vp, c_vp, c_vp, ctypes.c_int64, c_i32]),
    "dg_quantize_fp8": (c_i32, [c_vp, c_vp, c_vp, c_vp, ctypes.c_int64, c_i32]),
    "dg_quantize_fp8_lmhead": (c_i32, [c_vp, c_vp, c_vp, c_vp, ctypes.c_int64, c_i32]),
    "dg_prefill": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_i32]),
    "dg_ar_step": (c_i32, [c_vp, c_vp, c_i32, ctypes.POINTER(c_i32), c_vp, c_vp]),
    "dg_init_canvas": (c_i32, [c_vp, c_vp, ctypes.POINTER(DGStepArgs)]),
    "dg_denoise_step": (c_i32, [c_vp, c_vp, ctypes.POINTER(DGStepArgs)]),
    "dg_commit_block": (c_i32, [c_vp, c_vp, c_i32, ctypes.POINTER(c_i32), c_vp]),
    "dg_cache_len": (c_i32, [c_vp, c_i32]),
    "dg_reset": (c_i32, [c_vp, c_i32]),
    "dg_set_cache_len": (c_i32, [c_vp, c_i32, c_i32]),
    "dg_last_error": (ctypes.c_char_p, [c_vp]),
    "dg_sync": (c_i32, [c_vp, c_vp]),
    "dg_route_noalloc": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "dg_workspace_layout": (c_i32, [ctypes.POINTER(DGConfig), ctypes.POINTER(DGWsLayout)]),
    "dg_test_layer": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_vp, c_i32, c_i32]),
    "dg_test_route": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "dg_test_head": (c_i32, [c_vp, c_vp, ctypes.POINTER(DGStepArgs), c_vp]),
    "dg_test_forward": (c_i32, [c_vp, c_vp, ctypes.POINTER(DGStepArgs), c_vp, c_vp]),
    "dg_test_sample": (c_i32, [c_vp, c_vp, ctypes.POINTER(DGStepArgs), c_vp]),
    "dg_test_attention": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_vp, c_i32, c_i32, c_vp]),
    "dg_timing_enable": (c_i32, [c_vp, c_i32]),
    "dg_timing_read": (c_i32, [c_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i32), c_i32]),
}

# Words of the workspace "items" buffer (include/dg_test.h): expert-kernel
# waits that ran out (int32), and running routing statistics (uint64).
ITEMS_SPIN_TIMEOUTS = 409
ITEMS_TOUCHED_TOTAL = 410
ITEMS_PERMUTE_CALLS = 412
ROUTE_NOALLOC_MAX_ROWS = 2368  # DG_ROUTE_NOALLOC_MAX_ROWS (include/dg.h)

STAGES = ("embed", "norm", "qkv", "attn", "oproj", "router", "topk", "permute", "experts",
          "combine", "lmhead", "merge", "sampler", "selfcond")

_lib = None


def load() -> ctypes.CDLL:
    """Open libdg.so (built in-tree) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -m block_discrete_diffusion_dg_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class DGError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
