"""Float64 definitions of the weight-only quantized projection formats the pages run.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests, the smoke
check and the bench's CPU-baseline leg, never by the product path.

Sources:
  * hf2q 0.1.1, ``qwen3vl_text/forward.rs``, the dense FFN step: the gate, up and down
    weights of the converted Qwen3-VL checkpoints are GGML ``Q4_0`` tensors (as are the
    attention projections, per the same note's tensor count). The page names the type only;
    the layout taken here is GGML's published Q4_0 block: 32 consecutive weights of a row
    share one block of 18 bytes, a little-endian IEEE binary16 scale d followed by 16 bytes
    of 4-bit codes; byte j holds the code of weight j in its low nibble and of weight j + 16
    in its high nibble, and a code c stands for the weight d * (c - 8).
  * cortiq-engine 0.8.21, ``qwen3te.rs``: ``q8_exact_matmat`` / ``q8_dot4`` and the note on
    exact q8 projections above them: weight-only int8 rows, activations kept in f32, the row
    scale applied once per output, w[o, j] = row_scale[o] * q[o, j].

A projection with quantized weights is the ordinary product with the dequantized matrix,
x W^T; these functions define that matrix.
"""

import numpy as np

F64 = np.float64
Q4_0_BLOCK = 32          # weights per block
Q4_0_BYTES = 18          # 2-byte scale + 16 bytes of codes


def dequant_q4_0(blocks, rows, cols):
    """[rows, cols] float64 weights from Q4_0 blocks: a uint8 array of rows * cols / 32 blocks
    of 18 bytes, row-major (block b of row o covers columns 32b .. 32b + 31)."""
    if cols % Q4_0_BLOCK != 0:
        raise ValueError("Q4_0 needs cols to be a multiple of 32")
    nb = cols // Q4_0_BLOCK
    b = np.asarray(blocks, dtype=np.uint8).reshape(rows, nb, Q4_0_BYTES)
    d = b[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(F64)          # [rows, nb]
    qs = b[:, :, 2:]                                                   # [rows, nb, 16]
    low = (qs & 0x0F).astype(F64) - 8.0
    high = (qs >> 4).astype(F64) - 8.0
    codes = np.concatenate([low, high], axis=2)                        # weight j: low[j], j + 16: high[j]
    return (codes * d[:, :, None]).reshape(rows, cols)


def dequant_q8_row(q, row_scale):
    """[rows, cols] float64 weights row_scale[o] * q[o, j] from int8 codes [rows, cols]."""
    q = np.asarray(q, dtype=np.int8).astype(F64)
    return q * np.asarray(row_scale, dtype=F64)[:, None]


def dequant(fmt, data, rows, cols, row_scale=None):
    """Dispatch on the format name: "q4_0", "q8_row" or "dense" (data is the matrix)."""
    if fmt == "q4_0":
        return dequant_q4_0(data, rows, cols)
    if fmt == "q8_row":
        return dequant_q8_row(np.asarray(data).reshape(rows, cols), row_scale)
    if fmt == "dense":
        return np.asarray(data, dtype=F64).reshape(rows, cols)
    raise ValueError(f"unknown weight format {fmt}")
