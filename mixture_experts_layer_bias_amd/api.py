"""Python binding of the C ABI in include/moe_zc.h.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their device pointers and the current HIP stream are handed
to libmoe_zc.so.  Every step of the layer runs in the library's kernels; if
the library is missing this module raises (there is no fallback path).
PyTorch only provides device memory and streams.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import torch

from . import _lib

_DT = {torch.float32: _lib.MOE_ZC_F32, torch.bfloat16: _lib.MOE_ZC_BF16}
AUX_KEYS = ("logits", "topk_idx", "topk_gate", "loads", "offsets", "perm", "pos")


class MoeZcError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {moe_zc_status_string(code)} (status {code})")


def moe_zc_status_string(code: int) -> str:
    return _lib.load().moe_zc_status_string(int(code)).decode()


def moe_zc_abi_version() -> int:
    return int(_lib.load().moe_zc_abi_version())


def _dtype_code(dt) -> int:
    if isinstance(dt, int):
        return dt
    if isinstance(dt, str):
        return {"f32": _lib.MOE_ZC_F32, "bf16": _lib.MOE_ZC_BF16}[dt]
    return _DT[dt]


def moe_zc_workspace_size(T: int, d: int, I: int, N: int, Z: int, K: int, dtype) -> int:
    return int(_lib.load().moe_zc_workspace_size(T, d, I, N, Z, K, _dtype_code(dtype)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _aux_spec(T: int, N: int, Z: int, K: int, I: Optional[int] = None):
    E = N + Z
    spec = {"logits": ((T, E), torch.float32), "topk_idx": ((T, K), torch.int32),
            "topk_gate": ((T, K), torch.float32), "loads": ((E,), torch.int32),
            "offsets": ((N + 1,), torch.int32),
            "perm": ((max(1, T * min(K, N)),), torch.int32), "pos": ((T, K), torch.int32)}
    if I is not None:  # the saved pre-activations (a | u) of every grouped row
        spec["act"] = ((max(1, T * min(K, N)), 2 * I), torch.bfloat16)
    return spec


def alloc_aux(T: int, N: int, Z: int, K: int, device, keys=AUX_KEYS,
              I: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Caller-owned tensors for the optional outputs of moe_zc_forward; the
    key "act" (pre-activations, bf16 forwards) needs the hidden size I."""
    spec = _aux_spec(T, N, Z, K, I)
    if "act" in keys and I is None:
        raise ValueError("aux key 'act' needs I")
    return {k: torch.empty(*spec[k][0], dtype=spec[k][1], device=device) for k in keys}


class StageEvents:
    """HIP events recorded by moe_zc_forward at its stage boundaries."""

    def __init__(self):
        h = _lib.hip()
        self._ev = (ctypes.c_void_p * _lib.MOE_ZC_NUM_EVENTS)()
        for i in range(_lib.MOE_ZC_NUM_EVENTS):
            ev = ctypes.c_void_p()
            if h.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self._ev[i] = ev.value

    @property
    def array(self):
        return self._ev

    def stage_ms(self) -> Dict[str, float]:
        """Per-stage milliseconds of the last recorded forward (synchronises)."""
        h = _lib.hip()
        if h.hipEventSynchronize(self._ev[_lib.MOE_ZC_NUM_EVENTS - 1]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        out = {}
        for i, name in enumerate(_lib.STAGE_NAMES):
            ms = ctypes.c_float()
            if h.hipEventElapsedTime(ctypes.byref(ms), self._ev[i], self._ev[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = float(ms.value)
        return out

    def __del__(self):
        try:
            h = _lib.hip()
            for i in range(_lib.MOE_ZC_NUM_EVENTS):
                if self._ev[i]:
                    h.hipEventDestroy(self._ev[i])
        except Exception:
            pass


def _forward(name: str, x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
             weights, N: int, Z: int, K: int, I: int, residual, out, aux, workspace, events,
             fp8: bool = False):
    """Shared marshalling of the forward entry points; ``weights`` are the
    already checked weight tensors (or None).  The block-FP8 forward takes no
    dtype argument and has a workspace size of its own."""
    lib = _lib.load()
    T, d = x.shape
    dev = x.device
    dt = x.dtype
    E = N + Z
    _need(w_router, "w_router", torch.float32, (E, d), dev)
    _need(bias, "bias", torch.float32, (E,), dev)
    if residual is not None:
        _need(residual, "residual", dt, (T, d), dev)
    if out is None:
        out = torch.empty(T, d, dtype=dt, device=dev)
    _need(out, "out", dt, (T, d), dev)
    fn = getattr(lib, name)
    # weights: tensors (passed as pointers) and, for the FP8 forward, the
    # integer down-projection precision flag (passed as is)
    nulls = [w if isinstance(w, int) else None for w in weights]
    wargs = [w if isinstance(w, int) else _ptr(w) for w in weights]
    dt_arg = [] if fp8 else [_DT[dt]]
    need = (moe_zc_workspace_size_fp8(T, d, I, N, Z, K) if fp8
            else moe_zc_workspace_size(T, d, I, N, Z, K, dt))
    if need == 0:
        code = fn(None, None, None, *nulls, None, None, T, d, I, N, Z, K, *dt_arg, None, None, 0,
                  None)
        raise MoeZcError(code, name)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on x's device")
    a = _lib.MoeZcAux()
    if aux:
        spec = _aux_spec(T, N, Z, K, I)
        for k, t in aux.items():
            if k not in spec:
                raise ValueError(f"unknown aux key {k!r}")
            _need(t, f"aux[{k!r}]", spec[k][1], spec[k][0], dev)
            setattr(a, k, t.data_ptr())
    if events is not None:
        a.stage_events = ctypes.cast(events.array, ctypes.c_void_p).value
    code = fn(_ptr(x), _ptr(w_router), _ptr(bias), *wargs, _ptr(residual),
              _ptr(out), T, d, I, N, Z, K, *dt_arg, ctypes.byref(a), _ptr(workspace),
              workspace.numel(), _stream(dev))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, name)
    return out


def _check_x(x: torch.Tensor):
    if x.dim() != 2:
        raise ValueError("x must be [T, d]")
    if x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    if x.dtype not in _DT:
        raise ValueError(f"unsupported dtype {x.dtype}")
    _need(x, "x", x.dtype, tuple(x.shape), x.device)


def moe_zc_forward(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
                   w_gate: Optional[torch.Tensor], w_up: Optional[torch.Tensor],
                   w_down: Optional[torch.Tensor], N: int, Z: int, K: int,
                   residual: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None,
                   aux: Optional[Dict[str, torch.Tensor]] = None,
                   workspace: Optional[torch.Tensor] = None,
                   events: Optional[StageEvents] = None) -> torch.Tensor:
    """y = MoE-ZC(x) (+ residual); see include/moe_zc.h for the definition."""
    _check_x(x)
    T, d = x.shape
    dev, dt = x.device, x.dtype
    if N > 0:
        I = w_gate.shape[1]
        _need(w_gate, "w_gate", dt, (N, I, d), dev)
        _need(w_up, "w_up", dt, (N, I, d), dev)
        _need(w_down, "w_down", dt, (N, d, I), dev)
        weights = (w_gate, w_up, w_down)
    else:
        I = w_gate.shape[1] if w_gate is not None else 128
        weights = (None, None, None)
    return _forward("moe_zc_forward", x, w_router, bias, weights, N, Z, K, I, residual, out, aux,
                    workspace, events)


def moe_zc_packed_expert_bytes(d: int, I: int, dtype=torch.bfloat16):
    """(gate_up_bytes, down_bytes) of one expert's packed weights."""
    gu, dn = ctypes.c_size_t(), ctypes.c_size_t()
    code = _lib.load().moe_zc_packed_expert_bytes(d, I, _dtype_code(dtype), ctypes.byref(gu),
                                                  ctypes.byref(dn))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_packed_expert_bytes")
    return int(gu.value), int(dn.value)


def moe_zc_pack_expert_weights(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                               gate_up_packed: Optional[torch.Tensor] = None,
                               down_packed: Optional[torch.Tensor] = None):
    """Pack row-major bf16 expert weights ([n, I, d], [n, I, d], [n, d, I]) for
    moe_zc_forward_packed; returns (gate_up_packed, down_packed), uint8
    tensors of n * gate_up_bytes and n * down_bytes."""
    lib = _lib.load()
    n, I, d = w_gate.shape
    dev, dt = w_gate.device, w_gate.dtype
    if dev.type != "cuda":
        raise ValueError("weights must be GPU tensors")
    _need(w_gate, "w_gate", torch.bfloat16, (n, I, d), dev)
    _need(w_up, "w_up", torch.bfloat16, (n, I, d), dev)
    _need(w_down, "w_down", torch.bfloat16, (n, d, I), dev)
    gu, dn = moe_zc_packed_expert_bytes(d, I, dt)
    if gate_up_packed is None:
        gate_up_packed = torch.empty(n * gu, dtype=torch.uint8, device=dev)
    if down_packed is None:
        down_packed = torch.empty(n * dn, dtype=torch.uint8, device=dev)
    _need(gate_up_packed, "gate_up_packed", torch.uint8, (n * gu,), dev)
    _need(down_packed, "down_packed", torch.uint8, (n * dn,), dev)
    code = lib.moe_zc_pack_expert_weights(_ptr(w_gate), _ptr(w_up), _ptr(w_down), n, d, I,
                                          _DT[dt], _ptr(gate_up_packed), _ptr(down_packed),
                                          _stream(dev))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_pack_expert_weights")
    return gate_up_packed, down_packed


def moe_zc_forward_packed(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
                          gate_up_packed: Optional[torch.Tensor],
                          down_packed: Optional[torch.Tensor], N: int, Z: int, K: int, I: int,
                          residual: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None,
                          aux: Optional[Dict[str, torch.Tensor]] = None,
                          workspace: Optional[torch.Tensor] = None,
                          events: Optional[StageEvents] = None) -> torch.Tensor:
    """moe_zc_forward on weights packed by moe_zc_pack_expert_weights (bf16)."""
    _check_x(x)
    T, d = x.shape
    dev = x.device
    if N > 0:
        gu, dn = moe_zc_packed_expert_bytes(d, I, x.dtype)
        _need(gate_up_packed, "gate_up_packed", torch.uint8, (N * gu,), dev)
        _need(down_packed, "down_packed", torch.uint8, (N * dn,), dev)
        weights = (gate_up_packed, down_packed)
    else:
        weights = (None, None)
    return _forward("moe_zc_forward_packed", x, w_router, bias, weights, N, Z, K, I, residual,
                    out, aux, workspace, events)


def moe_zc_forward_packed_noalloc(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
                                  gate_up_packed: Optional[torch.Tensor],
                                  down_packed: Optional[torch.Tensor], N: int, Z: int, K: int,
                                  I: int, residual: Optional[torch.Tensor] = None,
                                  out: Optional[torch.Tensor] = None,
                                  aux: Optional[Dict[str, torch.Tensor]] = None,
                                  events: Optional[StageEvents] = None) -> torch.Tensor:
    """moe_zc_forward_packed with the library's fixed per-GPU scratch instead of
    a workspace (no allocation inside the call; ``out`` and ``aux`` must be
    given for the call as a whole to allocate nothing)."""
    _check_x(x)
    lib = _lib.load()
    T, d = x.shape
    dev, dt = x.device, x.dtype
    E = N + Z
    _need(w_router, "w_router", torch.float32, (E, d), dev)
    _need(bias, "bias", torch.float32, (E,), dev)
    if N > 0:
        gu, dn = moe_zc_packed_expert_bytes(d, I, dt)
        _need(gate_up_packed, "gate_up_packed", torch.uint8, (N * gu,), dev)
        _need(down_packed, "down_packed", torch.uint8, (N * dn,), dev)
    if residual is not None:
        _need(residual, "residual", dt, (T, d), dev)
    if out is None:
        out = torch.empty(T, d, dtype=dt, device=dev)
    _need(out, "out", dt, (T, d), dev)
    a = _lib.MoeZcAux()
    if aux:
        spec = _aux_spec(T, N, Z, K, I)
        for k, t in aux.items():
            if k not in spec:
                raise ValueError(f"unknown aux key {k!r}")
            _need(t, f"aux[{k!r}]", spec[k][1], spec[k][0], dev)
            setattr(a, k, t.data_ptr())
    if events is not None:
        a.stage_events = ctypes.cast(events.array, ctypes.c_void_p).value
    code = lib.moe_zc_forward_packed_noalloc(
        _ptr(x), _ptr(w_router), _ptr(bias), _ptr(gate_up_packed if N > 0 else None),
        _ptr(down_packed if N > 0 else None), _ptr(residual), _ptr(out), T, d, I, N, Z, K,
        _DT[dt], ctypes.byref(a), _stream(dev))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_forward_packed_noalloc")
    return out


def moe_zc_route(logits: torch.Tensor, bias: torch.Tensor, K: int,
                 topk_idx: Optional[torch.Tensor] = None,
                 topk_gate: Optional[torch.Tensor] = None,
                 loads: Optional[torch.Tensor] = None):
    """(topk_idx, topk_gate) from fp32 logits [T, E] and bias [E]; the expert
    loads [E] int32 are written into ``loads`` when it is given."""
    lib = _lib.load()
    T, E = logits.shape
    dev = logits.device
    _need(logits, "logits", torch.float32, (T, E), dev)
    _need(bias, "bias", torch.float32, (E,), dev)
    if topk_idx is None:
        topk_idx = torch.empty(T, K, dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty(T, K, dtype=torch.float32, device=dev)
    _need(topk_idx, "topk_idx", torch.int32, (T, K), dev)
    _need(topk_gate, "topk_gate", torch.float32, (T, K), dev)
    if loads is not None:
        _need(loads, "loads", torch.int32, (E,), dev)
    code = lib.moe_zc_route(_ptr(logits), _ptr(bias), T, E, K, _ptr(topk_idx), _ptr(topk_gate),
                            _ptr(loads), _stream(dev))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_route")
    return topk_idx, topk_gate


class PidState:
    """Gains (host) and error histories (device) of the bias controller."""

    def __init__(self, E: int, device, kp: float = 0.5, ki: float = 0.5, kd: float = 0.0):
        self.kp, self.ki, self.kd = float(kp), float(ki), float(kd)
        self.e_prev = torch.zeros(E, dtype=torch.float32, device=device)
        self.e_prev2 = torch.zeros(E, dtype=torch.float32, device=device)

    def as_struct(self) -> _lib.MoeZcPid:
        return _lib.MoeZcPid(self.kp, self.ki, self.kd, self.e_prev.data_ptr(),
                             self.e_prev2.data_ptr())


def moe_zc_bias_update(loads: torch.Tensor, target: torch.Tensor, bias: torch.Tensor,
                       pid: PidState) -> torch.Tensor:
    """One PID step on ``bias`` (in place) from ``loads``; returns ``bias``."""
    lib = _lib.load()
    E = bias.shape[0]
    dev = bias.device
    _need(loads, "loads", torch.int32, (E,), dev)
    _need(target, "target", torch.float32, (E,), dev)
    _need(bias, "bias", torch.float32, (E,), dev)
    _need(pid.e_prev, "pid.e_prev", torch.float32, (E,), dev)
    _need(pid.e_prev2, "pid.e_prev2", torch.float32, (E,), dev)
    st = pid.as_struct()
    code = lib.moe_zc_bias_update(_ptr(loads), _ptr(target), _ptr(bias), ctypes.byref(st), E,
                                  _stream(dev))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_bias_update")
    return bias


# ---- block-FP8 expert projections --------------------------------------------
def moe_zc_workspace_size_fp8(T: int, d: int, I: int, N: int, Z: int, K: int) -> int:
    return int(_lib.load().moe_zc_workspace_size_fp8(T, d, I, N, Z, K))


def moe_zc_packed_fp8_expert_bytes(d: int, I: int):
    """(gate_up_bytes, down_bytes) of one expert's packed FP8 weights."""
    gu, dn = ctypes.c_size_t(), ctypes.c_size_t()
    code = _lib.load().moe_zc_packed_fp8_expert_bytes(d, I, ctypes.byref(gu), ctypes.byref(dn))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_packed_fp8_expert_bytes")
    return int(gu.value), int(dn.value)


def moe_zc_pack_expert_weights_fp8(w_gate: torch.Tensor, w_up: torch.Tensor,
                                   w_down: Optional[torch.Tensor] = None,
                                   gate_up_fp8: Optional[torch.Tensor] = None,
                                   down_fp8: Optional[torch.Tensor] = None):
    """Quantize and pack bf16 gate/up weights ([n, I, d] each) for
    moe_zc_forward_packed_fp8; returns the uint8 tensor of n * gate_up_bytes,
    or (gate_up_fp8, down_fp8) when w_down ([n, d, I]) is given as well."""
    lib = _lib.load()
    n, I, d = w_gate.shape
    dev = w_gate.device
    if dev.type != "cuda":
        raise ValueError("weights must be GPU tensors")
    _need(w_gate, "w_gate", torch.bfloat16, (n, I, d), dev)
    _need(w_up, "w_up", torch.bfloat16, (n, I, d), dev)
    gu, dn = moe_zc_packed_fp8_expert_bytes(d, I)
    if gate_up_fp8 is None:
        gate_up_fp8 = torch.empty(n * gu, dtype=torch.uint8, device=dev)
    _need(gate_up_fp8, "gate_up_fp8", torch.uint8, (n * gu,), dev)
    if w_down is not None:
        _need(w_down, "w_down", torch.bfloat16, (n, d, I), dev)
        if down_fp8 is None:
            down_fp8 = torch.empty(n * dn, dtype=torch.uint8, device=dev)
        _need(down_fp8, "down_fp8", torch.uint8, (n * dn,), dev)
    elif down_fp8 is not None:
        raise ValueError("down_fp8 needs w_down")
    code = lib.moe_zc_pack_expert_weights_fp8(_ptr(w_gate), _ptr(w_up), _ptr(w_down), n, d, I,
                                              _ptr(gate_up_fp8), _ptr(down_fp8), _stream(dev))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_pack_expert_weights_fp8")
    return gate_up_fp8 if w_down is None else (gate_up_fp8, down_fp8)


def moe_zc_forward_packed_fp8(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
                              gate_up_fp8: Optional[torch.Tensor],
                              down: Optional[torch.Tensor], N: int, Z: int, K: int, I: int,
                              residual: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None,
                              aux: Optional[Dict[str, torch.Tensor]] = None,
                              workspace: Optional[torch.Tensor] = None,
                              events: Optional[StageEvents] = None,
                              down_fp8: bool = False) -> torch.Tensor:
    """moe_zc_forward (bf16) with the gate/up projection in block FP8:
    gate_up_fp8 from moe_zc_pack_expert_weights_fp8; ``down`` is the down half
    of moe_zc_pack_expert_weights (bf16), or with down_fp8 the FP8 down
    weights from moe_zc_pack_expert_weights_fp8."""
    _check_x(x)
    T, d = x.shape
    dev = x.device
    if x.dtype != torch.bfloat16:
        raise ValueError("the block-FP8 forward takes bf16 x")
    if N > 0:
        gu, dn8 = moe_zc_packed_fp8_expert_bytes(d, I)
        _, dn = moe_zc_packed_expert_bytes(d, I, x.dtype)
        _need(gate_up_fp8, "gate_up_fp8", torch.uint8, (N * gu,), dev)
        _need(down, "down", torch.uint8, (N * (dn8 if down_fp8 else dn),), dev)
        weights = (gate_up_fp8, down, int(bool(down_fp8)))
    else:
        weights = (None, None, int(bool(down_fp8)))
    return _forward("moe_zc_forward_packed_fp8", x, w_router, bias, weights, N, Z, K, I,
                    residual, out, aux, workspace, events, fp8=True)


def moe_zc_quantize_mx(x: torch.Tensor, codes: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None):
    """Block-FP8 codes [rows, d] and scale bytes [rows, d / 32] of bf16 x."""
    lib = _lib.load()
    if x.dim() != 2 or x.device.type != "cuda":
        raise ValueError("x must be a [rows, d] GPU tensor")
    rows, d = x.shape
    dev = x.device
    _need(x, "x", torch.bfloat16, (rows, d), dev)
    if codes is None:
        codes = torch.empty(rows, d, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(rows, max(d // 32, 1), dtype=torch.uint8, device=dev)
    _need(codes, "codes", torch.uint8, (rows, d), dev)
    _need(scales, "scales", torch.uint8, (rows, max(d // 32, 1)), dev)
    code = lib.moe_zc_quantize_mx(_ptr(x), rows, d, _ptr(codes), _ptr(scales), _stream(dev))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_quantize_mx")
    return codes, scales


# ---- backward ------------------------------------------------------------------
BWD_AUX_KEYS = ("logits", "topk_idx", "topk_gate", "offsets", "perm", "pos")


def moe_zc_backward_workspace_size(T: int, d: int, I: int, N: int, Z: int, K: int) -> int:
    return int(_lib.load().moe_zc_backward_workspace_size(T, d, I, N, Z, K))


def moe_zc_transposed_expert_bytes(d: int, I: int):
    """(gate_up_t_bytes, down_t_bytes) of one expert's packed transposed weights."""
    gu, dn = ctypes.c_size_t(), ctypes.c_size_t()
    code = _lib.load().moe_zc_transposed_expert_bytes(d, I, ctypes.byref(gu), ctypes.byref(dn))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_transposed_expert_bytes")
    return int(gu.value), int(dn.value)


def moe_zc_transpose_expert_weights(w_gate: torch.Tensor, w_up: torch.Tensor,
                                    w_down: torch.Tensor,
                                    w_gate_up_t: Optional[torch.Tensor] = None,
                                    w_down_t: Optional[torch.Tensor] = None):
    """Packed transposed expert weights for moe_zc_backward: returns
    (w_gate_up_t, w_down_t), uint8 tensors of n * gate_up_t_bytes and
    n * down_t_bytes ([W_gate; W_up]^T and W_down^T per expert)."""
    lib = _lib.load()
    n, I, d = w_gate.shape
    dev = w_gate.device
    if dev.type != "cuda":
        raise ValueError("weights must be GPU tensors")
    _need(w_gate, "w_gate", torch.bfloat16, (n, I, d), dev)
    _need(w_up, "w_up", torch.bfloat16, (n, I, d), dev)
    _need(w_down, "w_down", torch.bfloat16, (n, d, I), dev)
    gb, db = moe_zc_transposed_expert_bytes(d, I)
    if w_gate_up_t is None:
        w_gate_up_t = torch.empty(n * gb, dtype=torch.uint8, device=dev)
    if w_down_t is None:
        w_down_t = torch.empty(n * db, dtype=torch.uint8, device=dev)
    _need(w_gate_up_t, "w_gate_up_t", torch.uint8, (n * gb,), dev)
    _need(w_down_t, "w_down_t", torch.uint8, (n * db,), dev)
    code = lib.moe_zc_transpose_expert_weights(_ptr(w_gate), _ptr(w_up), _ptr(w_down), n, d, I,
                                               _ptr(w_gate_up_t), _ptr(w_down_t), _stream(dev))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_transpose_expert_weights")
    return w_gate_up_t, w_down_t


def moe_zc_backward(x: torch.Tensor, w_router: torch.Tensor, w_gate: Optional[torch.Tensor],
                    w_up: Optional[torch.Tensor], transposed, aux: Dict[str, torch.Tensor],
                    dy: torch.Tensor, N: int, Z: int, K: int, I: int,
                    out: Optional[Dict[str, torch.Tensor]] = None,
                    workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """Gradients of the layer for upstream gradient dy, replaying the routing
    the forward saved in ``aux`` (keys BWD_AUX_KEYS, plus "act" when the
    forward saved the pre-activations: then w_gate and w_up may be None);
    ``transposed`` is the pair from moe_zc_transpose_expert_weights (or None
    when N = 0).  Returns dx (bf16) and dw_router, dw_gate, dw_up, dw_down
    (fp32)."""
    lib = _lib.load()
    _check_x(x)
    T, d = x.shape
    dev = x.device
    E = N + Z
    if x.dtype != torch.bfloat16:
        raise ValueError("the backward takes bf16 x")
    _need(w_router, "w_router", torch.float32, (E, d), dev)
    _need(dy, "dy", torch.bfloat16, (T, d), dev)
    spec = _aux_spec(T, N, Z, K, I)
    for k in BWD_AUX_KEYS:
        if k not in aux:
            raise ValueError(f"aux lacks {k!r}")
        _need(aux[k], f"aux[{k!r}]", spec[k][1], spec[k][0], dev)
    act = aux.get("act")
    if act is not None:
        _need(act, "aux['act']", spec["act"][1], spec["act"][0], dev)
    shapes = {"dx": ((T, d), torch.bfloat16), "dw_router": ((E, d), torch.float32),
              "dw_gate": ((N, I, d), torch.float32), "dw_up": ((N, I, d), torch.float32),
              "dw_down": ((N, d, I), torch.float32)}
    out = dict(out or {})
    for k, (shp, dt) in shapes.items():
        if k not in out:
            out[k] = torch.empty(*shp, dtype=dt, device=dev)
        _need(out[k], k, dt, shp, dev)
    if N > 0:
        if act is None or w_gate is not None:
            _need(w_gate, "w_gate", torch.bfloat16, (N, I, d), dev)
        if act is None or w_up is not None:
            _need(w_up, "w_up", torch.bfloat16, (N, I, d), dev)
        gut, dnt = transposed
        gb, db = moe_zc_transposed_expert_bytes(d, I)
        _need(gut, "w_gate_up_t", torch.uint8, (N * gb,), dev)
        _need(dnt, "w_down_t", torch.uint8, (N * db,), dev)
        weights = (w_gate, w_up, gut, dnt)
    else:
        weights = (None, None, None, None)
    need = moe_zc_backward_workspace_size(T, d, I, N, Z, K)
    a = _lib.MoeZcAux()
    for k in BWD_AUX_KEYS:
        setattr(a, k, aux[k].data_ptr())
    if act is not None:
        a.act = act.data_ptr()
    if need == 0:
        code = lib.moe_zc_backward(None, None, None, None, None, None, ctypes.byref(a), None, None,
                                   None, None, None, None, T, d, I, N, Z, K, None, 0, None)
        raise MoeZcError(code, "moe_zc_backward")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on x's device")
    code = lib.moe_zc_backward(_ptr(x), _ptr(w_router), *[_ptr(w) for w in weights],
                               ctypes.byref(a), _ptr(dy), _ptr(out["dx"]), _ptr(out["dw_router"]),
                               _ptr(out["dw_gate"]), _ptr(out["dw_up"]), _ptr(out["dw_down"]),
                               T, d, I, N, Z, K, _ptr(workspace), workspace.numel(), _stream(dev))
    if code != _lib.MOE_ZC_OK:
        raise MoeZcError(code, "moe_zc_backward")
    return out
