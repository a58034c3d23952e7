"""Expert weights and the SwiGLU expert in fp64 (oracle).

The slot is a complete expert and the host bank of an expert is byte-identical
to its device slot (snackonai, "The Architecture, Unpacked", first decision).
Bank layout (row-major matrices, contraction axis contiguous):
  f32  : W_gate[I][H] | W_up[I][H] | W_down[H][I]
  bf16 : same, bfloat16
  mxfp4: codes W_gate[I][H/2] | W_up[I][H/2] | W_down[H][I/2], then
         scales W_gate[I][H/32] | W_up[I][H/32] | W_down[H][I/32];
         OCP MX v1.0 e2m1 elements (two per byte, low nibble first) with one
         e8m0 scale per 32 contraction elements.
The expert is SwiGLU with no biases: p = W_down (silu(W_gate x) * (W_up x)),
silu(z) = z / (1 + e^-z).  The pages name neither the FFN form nor the
formats' arithmetic; the merged result must equal the checkpoint's own
computation exactly (snackonai, "What It Actually Does"), so the oracle
evaluates the dequantised values of the exact bytes in fp64.
"""
from __future__ import annotations

import numpy as np


def expert_bytes(w_dtype: str, H: int, I: int) -> int:
    if w_dtype == "f32":
        return 12 * H * I
    if w_dtype == "bf16":
        return 6 * H * I
    if w_dtype == "mxfp4":
        return 3 * H * I // 2 + 3 * H * I // 32
    raise ValueError(w_dtype)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e2m1_value(code: int) -> float:
    """OCP MX FP4 (E2M1): sign bit 3, exponent bits 2..1 (bias 1), mantissa
    bit 0; exponent field 0 is subnormal (0 or 0.5)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + 0.5 * m)
    return -mag if s else mag


def e8m0_value(byte: int) -> float:
    """OCP MX E8M0 scale: 2^(byte - 127); 0xFF is NaN."""
    return float("nan") if byte == 0xFF else 2.0 ** (int(byte) - 127)


_E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E8M0 = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)
# the two elements a code byte holds, (low nibble, high nibble) = (even, odd)
_E2M1_PAIR = np.stack([_E2M1[np.arange(256) & 0x0F], _E2M1[np.arange(256) >> 4]], axis=-1)


def mxfp4_matrix(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Dequantise a rows x cols MXFP4 matrix (contraction axis = cols): each
    code byte gives elements 2i (low nibble) and 2i+1 (high nibble), and each
    run of 32 elements along a row is multiplied by its E8M0 scale."""
    c = np.asarray(codes, np.uint8).reshape(rows, cols // 2)
    s = np.asarray(scales, np.uint8).reshape(rows, cols // 32)
    vals = _E2M1_PAIR[c].reshape(rows, cols // 32, 32)
    vals *= _E8M0[s][:, :, None]
    return vals.reshape(rows, cols)


def expert_weights(raw: np.ndarray, w_dtype: str, H: int, I: int):
    """Decode one bank into (W_gate [I,H], W_up [I,H], W_down [H,I]) fp64."""
    raw = np.asarray(raw, np.uint8)
    nb = expert_bytes(w_dtype, H, I)
    assert raw.size >= nb
    raw = raw[:nb]
    if w_dtype == "f32":
        v = raw.view(np.float32).astype(np.float64)
        return (v[:I * H].reshape(I, H), v[I * H:2 * I * H].reshape(I, H),
                v[2 * I * H:].reshape(H, I))
    if w_dtype == "bf16":
        v = bf16_to_f64(raw.view(np.uint16))
        return (v[:I * H].reshape(I, H), v[I * H:2 * I * H].reshape(I, H),
                v[2 * I * H:].reshape(H, I))
    o = 0
    cg = raw[o:o + I * H // 2]; o += I * H // 2
    cu = raw[o:o + I * H // 2]; o += I * H // 2
    cd = raw[o:o + H * I // 2]; o += H * I // 2
    sg = raw[o:o + I * H // 32]; o += I * H // 32
    su = raw[o:o + I * H // 32]; o += I * H // 32
    sd = raw[o:o + H * I // 32]
    return (mxfp4_matrix(cg, sg, I, H), mxfp4_matrix(cu, su, I, H), mxfp4_matrix(cd, sd, H, I))


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def ffn(x: np.ndarray, w) -> np.ndarray:
    """SwiGLU expert on rows x [T, H] (fp64) -> [T, H]."""
    wg, wu, wd = w
    x = np.asarray(x, np.float64)
    g = x @ wg.T
    u = x @ wu.T
    return (silu(g) * u) @ wd.T
