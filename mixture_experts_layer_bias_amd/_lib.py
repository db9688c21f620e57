"""ctypes view of libmoe_zc.so (declarations mirror include/moe_zc.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_zc.so")

MOE_ZC_OK = 0
MOE_ZC_ERR_INVALID = 1
MOE_ZC_ERR_WORKSPACE = 2
MOE_ZC_ERR_UNSUPPORTED = 3
MOE_ZC_ERR_HIP = 4
MOE_ZC_F32 = 0
MOE_ZC_BF16 = 1
MOE_ZC_NUM_STAGES = 8
MOE_ZC_NUM_EVENTS = 9
STAGE_NAMES = ("router_gemm", "softmax_topk", "chunk_hist", "scan", "permute",
               "gemm_gate_up_swiglu", "gemm_down", "combine")

# every symbol include/moe_zc.h declares
EXPORTS = ("moe_zc_workspace_size", "moe_zc_forward", "moe_zc_packed_expert_bytes",
           "moe_zc_pack_expert_weights", "moe_zc_forward_packed", "moe_zc_route",
           "moe_zc_bias_update", "moe_zc_status_string", "moe_zc_abi_version",
           "moe_zc_packed_fp8_expert_bytes", "moe_zc_pack_expert_weights_fp8",
           "moe_zc_workspace_size_fp8", "moe_zc_forward_packed_fp8", "moe_zc_quantize_mx",
           "moe_zc_transpose_expert_weights", "moe_zc_backward_workspace_size",
           "moe_zc_backward", "moe_zc_transposed_expert_bytes",
           "moe_zc_forward_packed_noalloc")
MOE_ZC_NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeZcAux(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_idx", ctypes.c_void_p),
                ("topk_gate", ctypes.c_void_p), ("loads", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("pos", ctypes.c_void_p), ("stage_events", ctypes.c_void_p),
                ("act", ctypes.c_void_p)]


class MoeZcPid(ctypes.Structure):
    _fields_ = [("kp", ctypes.c_float), ("ki", ctypes.c_float), ("kd", ctypes.c_float),
                ("e_prev", ctypes.c_void_p), ("e_prev2", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    """The built library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m mixture_experts_layer_bias_amd._build` (there is no "
            "non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.moe_zc_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.c_int]
    lib.moe_zc_workspace_size.restype = sz
    lib.moe_zc_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                   i32, ctypes.c_int, ctypes.POINTER(MoeZcAux), vp, sz, vp]
    lib.moe_zc_forward.restype = ctypes.c_int
    lib.moe_zc_packed_expert_bytes.argtypes = [i64, i64, ctypes.c_int, ctypes.POINTER(sz),
                                               ctypes.POINTER(sz)]
    lib.moe_zc_packed_expert_bytes.restype = ctypes.c_int
    lib.moe_zc_pack_expert_weights.argtypes = [vp, vp, vp, i32, i64, i64, ctypes.c_int, vp, vp,
                                               vp]
    lib.moe_zc_pack_expert_weights.restype = ctypes.c_int
    lib.moe_zc_forward_packed.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                          i32, ctypes.c_int, ctypes.POINTER(MoeZcAux), vp, sz, vp]
    lib.moe_zc_forward_packed.restype = ctypes.c_int
    lib.moe_zc_forward_packed_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32,
                                                  i32, i32, ctypes.c_int,
                                                  ctypes.POINTER(MoeZcAux), vp]
    lib.moe_zc_forward_packed_noalloc.restype = ctypes.c_int
    lib.moe_zc_packed_fp8_expert_bytes.argtypes = [i64, i64, ctypes.POINTER(sz),
                                                   ctypes.POINTER(sz)]
    lib.moe_zc_packed_fp8_expert_bytes.restype = ctypes.c_int
    lib.moe_zc_pack_expert_weights_fp8.argtypes = [vp, vp, vp, i32, i64, i64, vp, vp, vp]
    lib.moe_zc_pack_expert_weights_fp8.restype = ctypes.c_int
    lib.moe_zc_workspace_size_fp8.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.moe_zc_workspace_size_fp8.restype = sz
    lib.moe_zc_forward_packed_fp8.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i64, i64, i64,
                                              i32, i32, i32, ctypes.POINTER(MoeZcAux), vp, sz,
                                              vp]
    lib.moe_zc_forward_packed_fp8.restype = ctypes.c_int
    lib.moe_zc_quantize_mx.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.moe_zc_quantize_mx.restype = ctypes.c_int
    lib.moe_zc_transpose_expert_weights.argtypes = [vp, vp, vp, i32, i64, i64, vp, vp, vp]
    lib.moe_zc_transpose_expert_weights.restype = ctypes.c_int
    lib.moe_zc_transposed_expert_bytes.argtypes = [i64, i64, ctypes.POINTER(sz),
                                                   ctypes.POINTER(sz)]
    lib.moe_zc_transposed_expert_bytes.restype = ctypes.c_int
    lib.moe_zc_backward_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.moe_zc_backward_workspace_size.restype = sz
    lib.moe_zc_backward.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(MoeZcAux), vp, vp, vp,
                                    vp, vp, vp, i64, i64, i64, i32, i32, i32, vp, sz, vp]
    lib.moe_zc_backward.restype = ctypes.c_int
    lib.moe_zc_route.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, vp]
    lib.moe_zc_route.restype = ctypes.c_int
    lib.moe_zc_bias_update.argtypes = [vp, vp, vp, ctypes.POINTER(MoeZcPid), i32, vp]
    lib.moe_zc_bias_update.restype = ctypes.c_int
    lib.moe_zc_status_string.argtypes = [ctypes.c_int]
    lib.moe_zc_status_string.restype = ctypes.c_char_p
    lib.moe_zc_abi_version.argtypes = []
    lib.moe_zc_abi_version.restype = i32
    _lib = lib
    return lib


# ---- HIP events (timing plumbing; the HIP runtime is already loaded) --------
_hip = None


def hip() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        h = None
        for name in ("libamdhip64.so", "libamdhip64.so.7", "/opt/rocm/lib/libamdhip64.so"):
            try:
                h = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if h is None:
            raise ImportError("libamdhip64.so not found")
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventCreate.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.restype = ctypes.c_int
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.restype = ctypes.c_int
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        h.hipEventElapsedTime.restype = ctypes.c_int
        _hip = h
    return _hip
