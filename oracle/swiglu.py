"""Fused SwiGLU + re-quantisation (oracle; test infrastructure only).

HALOps "GEMM" page, fused_swiglu_quant section: the input row is
[gate | up] (gate = first half of the columns, up = second half) and
y = up * silu(gate) = up * gate / (1 + exp(-gate)); y is then quantised
group-wise.  Only the first token_nums_per_expert[e] rows of each expert's
slot are processed.

Readings (the page leaves these open):
  * y is formed in float64 here, from the BF16 inputs, with no intermediate
    BF16 rounding (the op is a single pass).
  * The output encoding follows the library mode: MXFP8 (E4M3, UE8M0 per 32),
    MXFP4 (E2M1, UE8M0 per 32) or NVFP4 (E2M1, UE4M3 per 16 with a supplied
    FP32 global scale).
  * Rows outside every group, and rows of a group beyond its valid count, are
    not written.
Because exp() differs between implementations, several code tensors can be
correct for one input.  The quantisation itself is exact and is checked
bit-for-bit on the FP32 y that the device produced; y is checked against
``swiglu_f64`` within a relative tolerance.
"""

import numpy as np

from . import formats as F
from . import quant as Q


def swiglu_values_f64(gate, up):
    """y = up * gate / (1 + exp(-gate)) of real gate / up values, float64."""
    gate = np.asarray(gate, np.float64)
    up = np.asarray(up, np.float64)
    with np.errstate(over="ignore"):
        return up * gate / (1.0 + np.exp(-gate))


def swiglu_f64(x_bits, h):
    """y[r, j] = up[r, j] * gate[r, j] / (1 + exp(-gate[r, j])) in float64."""
    x = F.bf16_decode(x_bits)
    return swiglu_values_f64(x[:, :h], x[:, h:2 * h])


def processed_rows(rows, group_end=None, slot_rows=0, valid=None, num_groups=0):
    """Boolean mask of the rows the fused op writes.

    Contiguous form: group g spans [end[g-1], end[g]) (ends clamped to
    [previous end, rows]).  Slot form: group g spans
    [g*slot_rows, (g+1)*slot_rows).  In both forms only the first
    min(valid[g], size) rows are processed when ``valid`` is given."""
    mask = np.zeros(rows, dtype=bool)
    if group_end is not None:
        prev = 0
        for g, end in enumerate(np.asarray(group_end, dtype=np.int64)):
            hi = int(min(max(int(end), prev), rows))
            size = hi - prev
            c = size if valid is None else int(min(max(int(valid[g]), 0), size))
            mask[prev:prev + c] = True
            prev = hi
    else:
        for g in range(num_groups):
            lo = g * slot_rows
            size = max(0, min(slot_rows, rows - lo))
            c = size if valid is None else int(min(max(int(valid[g]), 0), size))
            mask[lo:lo + c] = True
    return mask


def quantize_y(y, mode, g=None):
    """The group-wise quantisation applied to y (float64 holding exact FP32
    values for NVFP4).  Returns (codes, sf)."""
    if mode in ("mxfp8", "mxfp4"):
        return Q.mx_quant_values(y, mode)
    if mode == "nvfp4":
        codes, sf, _ = Q.nvfp4_quant_values(y, g)
        return codes, sf
    raise ValueError(mode)


def swiglu_quant(x_bits, h, mode, mask=None, g=None):
    """Full oracle: SwiGLU in float64, then quantisation of the processed rows.
    NVFP4 quantises y rounded once to FP32 (its recipe is defined on FP32
    values).  Returns (codes, sf, y) over the masked rows only."""
    y = swiglu_f64(x_bits, h)
    if mask is not None:
        y = y[mask]
    if mode == "nvfp4":
        y = y.astype(np.float32).astype(np.float64)
    codes, sf = quantize_y(y, mode, g)
    return codes, sf, y
