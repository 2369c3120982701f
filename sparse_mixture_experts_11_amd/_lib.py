"""ctypes view of libmoe.so (the C ABI declared in include/moe.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 = 0, 1, 2, 3
MOE_GATE_RENORM, MOE_GATE_PROB = 0, 1
MOE_ACT_SWIGLU, MOE_ACT_SITU_GLU = 0, 1
MOE_STATIC_SCRATCH_BYTES = 64 << 20   # moe_forward_noalloc's per-GPU scratch

# Every symbol include/moe.h declares.
EXPORTS = ("moe_desc_init", "moe_status_string", "moe_workspace_bytes",
           "moe_capacity_from_factor", "moe_route", "moe_route_biased", "moe_qb_update",
           "moe_route_backward", "moe_backward_workspace_bytes", "moe_experts_backward",
           "moe_latent_backward",
           "moe_dispatch", "moe_expert_ffn", "moe_expert_ffn_scaled",
           "moe_combine",
           "moe_forward", "moe_forward_noalloc", "moe_forward_traced", "moe_stage_name")


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("h", ctypes.c_int32),
                ("N", ctypes.c_int32), ("k", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("act", ctypes.c_int32), ("beta_g", ctypes.c_float), ("beta_u", ctypes.c_float),
                ("l", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("h_shared", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("aux_alpha", ctypes.c_float)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("W_route", "W_gate", "W_up", "W_down", "W_ldown",
                                                "W_lup", "Ws_gate", "Ws_up", "Ws_down",
                                                "selection_bias", "gate_scale", "up_scale",
                                                "down_scale")]


class MoeOutputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_idx", "topk_w", "stats", "counts",
                                                "offsets", "kept_offsets", "perm", "row_of",
                                                "drop", "y_perm", "gate_up")]


class MoeLatentGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("du", "dz", "dW_route", "dW_ldown", "dW_lup",
                                                "dW_gate", "dW_up", "dW_down", "dWs_gate",
                                                "dWs_up", "dWs_down")]


class LibraryMissing(RuntimeError):
    pass


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so; raise loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(SO_PATH):
        raise LibraryMissing(f"{SO_PATH} not found: build it first "
                             "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(SO_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(MoeDesc)
    lib.moe_desc_init.argtypes = [D]
    lib.moe_desc_init.restype = None
    lib.moe_status_string.argtypes = [I32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_workspace_bytes.argtypes = [D, ctypes.POINTER(SZ)]
    lib.moe_workspace_bytes.restype = I32
    lib.moe_capacity_from_factor.argtypes = [I64, I32, I32, ctypes.c_double]
    lib.moe_capacity_from_factor.restype = I32
    lib.moe_route.argtypes = [D, P, P, P, P, P, P, SZ, P]
    lib.moe_route.restype = I32
    lib.moe_route_biased.argtypes = [D, P, P, P, P, P, P, P, SZ, P]
    lib.moe_route_biased.restype = I32
    lib.moe_qb_update.argtypes = [D, P, P, P, I32, I32, P, P, SZ, P]
    lib.moe_qb_update.restype = I32
    lib.moe_route_backward.argtypes = [D, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, SZ, P]
    lib.moe_route_backward.restype = I32
    lib.moe_backward_workspace_bytes.argtypes = [D, ctypes.POINTER(SZ)]
    lib.moe_backward_workspace_bytes.restype = I32
    lib.moe_experts_backward.argtypes = [D, ctypes.c_void_p] + [P] * 13 + [SZ, P]
    lib.moe_experts_backward.restype = I32
    lib.moe_latent_backward.argtypes = [D, ctypes.POINTER(MoeWeights), P,
                                        ctypes.POINTER(MoeOutputs), P, ctypes.c_float,
                                        ctypes.POINTER(MoeLatentGrads), P, SZ, P]
    lib.moe_latent_backward.restype = I32
    lib.moe_dispatch.argtypes = [D, P, P, P, P, P, P, P, P, SZ, P]
    lib.moe_dispatch.restype = I32
    lib.moe_expert_ffn.argtypes = [D, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.moe_expert_ffn.restype = I32
    lib.moe_expert_ffn_scaled.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.moe_expert_ffn_scaled.restype = I32
    lib.moe_combine.argtypes = [D, P, P, P, P, P]
    lib.moe_combine.restype = I32
    lib.moe_forward.argtypes = [D, ctypes.POINTER(MoeWeights), P, P,
                                ctypes.POINTER(MoeOutputs), P, SZ, P]
    lib.moe_forward.restype = I32
    lib.moe_forward_noalloc.argtypes = [D, ctypes.POINTER(MoeWeights), P, P,
                                        ctypes.POINTER(MoeOutputs), P]
    lib.moe_forward_noalloc.restype = I32
    lib.moe_forward_traced.argtypes = [D, ctypes.POINTER(MoeWeights), P, P,
                                       ctypes.POINTER(MoeOutputs), P, SZ, P,
                                       ctypes.POINTER(ctypes.c_void_p), I32]
    lib.moe_forward_traced.restype = I32
    lib.moe_stage_name.argtypes = [D, I32, ctypes.POINTER(I32)]
    lib.moe_stage_name.restype = ctypes.c_char_p
    _lib = lib
    return lib
