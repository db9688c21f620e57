"""FP8 block quantization for the mixed-precision expert path (fp64 oracle).

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.

The pages say LongCat-Flash quantizes with the same fine-grained block scheme
as DeepSeek-V3, mixed per layer: the down projection's input activations reach
magnitudes near 1e6 and some expert layers show large block-FP8 error, so
precision is chosen layer by layer
(『衝上熱搜！美團大模型，靠「快」火了』, section on system-level optimisation,
paragraph on quantization).

Readings (the pages name the scheme but define no format):
  * format: FP8 E4M3 elements (1 sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent field 0 holds subnormals, code 0x7F is NaN, the
    largest finite magnitude is 448), one power-of-two scale per block of 32
    consecutive values along the reduction axis, stored as an 8-bit biased
    exponent (E8M0, bias 127).  This is the block-scaled FP8 the MI355X matrix
    cores consume;
  * scale: the smallest power of two 2^s with amax <= 448 * 2^s, i.e.
    DeepSeek-style amax scaling rounded up to a power of two, so no element
    saturates; s is clamped to [-127, 127]; an all-zero block takes s = -127;
  * rounding: round to nearest, ties to even, onto the E4M3 grid;
  * mixed precision: the gate/up projection runs in FP8 (x quantized per
    token per 32 channels, W_gate and W_up per output row per 32 inputs); the
    down projection stays bf16 by default, since its input is where the pages
    find the extreme activations, and is FP8 as a per-layer option
    (down_fp8): the hidden activation h = silu(a) * u of each grouped row is
    quantized per row in blocks of 32 along I, W_down per output row in
    blocks of 32 along I, and o = dequant(h) dequant(W_down)^T.  Precision is
    a per-layer choice on the pages, so both settings are offered.

Pins (tests/pins.py): every code decodes by the closed form of the format and
re-encodes to itself; rounding of arbitrary values equals a brute-force
nearest search over the 127 finite non-negative codes with ties to the even
code; the scale is the minimal one (closed form); the quantization error is
within half a step; quantization is lossless for values already on a block's
grid, where the FP8 layer equals the bf16 layer exactly.  The FP8 down
projection (down_projection_fp8) is lossless when h and W_down lie on their
block grids along I, and a hand-worked block (scale 2^0, a tie rounded to
the even code, a value rounded down) gives the products written out by hand
(tests/golden/fp8_down_example.json).
"""
from __future__ import annotations

import numpy as np

from . import moe_zc as _layer

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte (NaN for 0x7F / 0xFF), by the format's closed form."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode(y) -> np.ndarray:
    """Round-to-nearest-even onto the E4M3 grid; |y| must not exceed 448.
    The sign bit is copied from y.

    Subnormals (|y| < 2^-6) are multiples of 2^-9: code = rint(|y| 2^9), and a
    result of 8 is exactly the first normal code.  A normal |y| = m 2^E
    (1 <= m < 2) has code 8 (E + 7) + rint(8 (m - 1)); a mantissa that rounds
    up to 8 carries into the exponent field, which is the next binade's first
    code.  Both pieces are exact in fp64."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(a > E4M3_MAX) or np.any(~np.isfinite(a)):
        raise ValueError("value outside the E4M3 range")
    sub = a < 2.0 ** -6
    m, ex = np.frexp(np.where(sub, 1.0, a))          # a = m 2^ex, 0.5 <= m < 1
    E = ex - 1                                       # a = (2m) 2^E, 1 <= 2m < 2
    code_n = 8 * (E + 7) + np.rint(8.0 * (2.0 * m - 1.0))
    code_s = np.rint(a * 2.0 ** 9)
    code = np.where(sub, code_s, code_n).astype(np.int64)
    # the sign bit is the input's, also for -0 and for values rounding to 0
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def mx_scale_exponent(amax) -> np.ndarray:
    """Smallest integer s with amax <= 448 * 2^s, clamped to [-127, 127]
    (amax = 0 gives -127).  With amax = f 2^E (1 <= f < 2): s = E - 8 when
    f <= 1.75 and E - 7 otherwise, since 448 = 1.75 * 2^8."""
    a = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(np.where(a > 0, a, 1.0))
    E = ex - 1
    s = E - 8 + (2.0 * m > 1.75)
    s = np.where(a > 0, s, -127)
    return np.clip(s, -127, 127).astype(np.int64)


def mx_quantize(v, axis=-1):
    """Block quantization along ``axis`` in blocks of 32 (the axis length must
    be a multiple of 32).  Returns (codes uint8, same shape as v; scales uint8
    E8M0 = s + 127, shape with that axis divided by 32)."""
    v = np.moveaxis(_layer._f64(v), axis, -1)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError("axis length must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    s = mx_scale_exponent(np.abs(blk).max(axis=-1))
    codes = e4m3_encode(blk * np.ldexp(1.0, -s)[..., None])
    codes = np.moveaxis(codes.reshape(v.shape), -1, axis)
    scales = np.moveaxis((s + 127).astype(np.uint8), -1, axis)
    return codes, scales


def mx_dequantize(codes, scales, axis=-1) -> np.ndarray:
    c = np.moveaxis(np.asarray(codes), axis, -1)
    sc = np.moveaxis(np.asarray(scales, dtype=np.int64), axis, -1)
    # the closed form evaluated once per code value (256 of them), then looked up
    table = e4m3_decode(np.arange(256, dtype=np.uint8))
    vals = table[np.asarray(c, dtype=np.uint8)].reshape(c.shape[:-1] + (c.shape[-1] // BLOCK, BLOCK))
    out = vals * np.ldexp(1.0, sc - 127)[..., None]
    return np.moveaxis(out.reshape(c.shape), -1, axis)


def down_projection_fp8(h, w_down) -> np.ndarray:
    """o = dequant(quant(h)) dequant(quant(W_down))^T for hidden rows h [m, I]
    and W_down [d, I]: both quantized along I (the reduction axis) in blocks
    of 32, h per row, W_down per output row."""
    h_dq = mx_dequantize(*mx_quantize(h, axis=-1), axis=-1)
    wd_dq = mx_dequantize(*mx_quantize(w_down, axis=-1), axis=-1)
    return h_dq @ wd_dq.T


def forward_tokens_fp8(x_rows, logits32_rows, bias, get_expert, N: int, K: int,
                       residual_rows=None, down_fp8: bool = False):
    """Layer output for a set of tokens with the gate/up projection in block
    FP8, given their fp32 logits.  x is quantized per token, so any subset of
    tokens can be evaluated alone; get_expert(e) returns the bf16 (W_gate[e],
    W_up[e], W_down[e]), of which gate and up are quantized per output row.
    With down_fp8 the down projection runs in block FP8 as well
    (down_projection_fp8 on the fp64 hidden activation).  The identity
    experts pass x itself (they compute nothing)."""
    x64 = _layer._f64(x_rows)
    xq, xs = mx_quantize(x64, axis=-1)
    x_dq = mx_dequantize(xq, xs, axis=-1)
    rt = _layer.route(logits32_rows, bias, K, N)
    idx, g = rt["idx"], rt["gate"]
    T = x64.shape[0]
    rows = np.zeros((T, K, x64.shape[1]))
    for e in np.unique(idx[idx < N]):
        tt, kk = np.nonzero(idx == e)
        wg, wu, wd = (_layer._f64(w) for w in get_expert(int(e)))
        wg = mx_dequantize(*mx_quantize(wg, axis=-1), axis=-1)
        wu = mx_dequantize(*mx_quantize(wu, axis=-1), axis=-1)
        if down_fp8:
            a = x_dq[tt] @ wg.T
            u = x_dq[tt] @ wu.T
            rows[tt, kk] = down_projection_fp8(_layer.silu(a) * u, wd)
        else:
            # gate/up on the dequantized FP8 operands, down on the bf16 weights
            rows[tt, kk] = _layer.swiglu_ffn(x_dq[tt], wg, wu, wd)
    y = _layer.combine(x64, idx, g, rows, N, residual_rows)
    return y, rt


def forward_fp8_gateup(x, w_router, bias, w_gate, w_up, w_down, N: int, Z: int, K: int,
                       residual=None, logits32=None, down_fp8: bool = False):
    """The whole layer with the gate/up projection in block FP8, and the down
    projection too with ``down_fp8`` (see forward_tokens_fp8); routing uses
    ``logits32`` when given, otherwise the fp64 logits rounded once to fp32
    (the router itself is not quantized)."""
    l64 = _layer.router_logits(x, w_router)
    if logits32 is None:
        logits32 = l64.astype(np.float32)

    def get(e):
        return w_gate[e], w_up[e], w_down[e]

    y, rt = forward_tokens_fp8(x, logits32, bias, get, N, K, residual, down_fp8=down_fp8)
    rt["logits64"] = l64
    rt["y"] = y
    return rt
