"""The oracle's view of one DiT block on a set of token rows (test helper).

Rows are independent through every step of a block (per-token
quantization, per-row GEMM outputs, element-wise SiLU/SwiGLU), so the
oracle evaluated on a few rows of the block input gives exactly those rows
of every intermediate and output the device computes on the whole input.
The data flow is the one ``w8a8_int8_gemm_amd.block.BlockRunner`` runs.
"""
from __future__ import annotations

import numpy as np


def block_rows(orc, x_rows: np.ndarray, params: dict, mlp: str = "silu",
               o_input: str = "x") -> dict:
    """Oracle of one block on ``x_rows`` (BF16 bits [R, H]).

    Returns the codes and scales of the block input (``xq``, ``xs``), the
    BF16 outputs of the six projections, the codes and scales of the FC2
    input (``hq``, ``hs``) and, when the attention output projection reads
    V's output, that input's codes and scales (``oq``, ``os``)."""
    out = {}
    out["xq"], out["xs"] = orc.quantize_act(x_rows)
    for n in ("q", "k", "v", "fc1"):
        p = params[n]
        out[n] = orc.linear(x_rows, p.w, p.sw, p.bias)
    o_in = out["v"] if o_input == "v" else x_rows
    if o_input == "v":
        out["oq"], out["os"] = orc.quantize_act(o_in)
    p = params["o"]
    out["o"] = orc.linear(o_in, p.w, p.sw, p.bias)
    h = (orc.swiglu_bf16(out["fc1"]) if mlp == "swiglu"
         else orc.silu_bf16(out["fc1"]))
    out["hq"], out["hs"] = orc.quantize_act(h)
    p = params["fc2"]
    out["fc2"] = orc.linear(h, p.w, p.sw, p.bias)
    return out


def tile_rows(M: int, tile: int = 256, salt: int = 0) -> np.ndarray:
    """One token row from every ``tile``-row token tile, at an offset inside
    the tile that changes from tile to tile (so the rows visit many
    positions within a tile), plus the first and the last row."""
    rows = {0, M - 1}
    for t in range((M + tile - 1) // tile):
        lo = t * tile
        n = min(M, lo + tile) - lo
        rows.add(lo + (t * 97 + 13 + salt) % n)
    return np.array(sorted(rows), np.int64)


def spread_rows(M: int, count: int, salt: int = 0) -> np.ndarray:
    """About ``count`` rows spread evenly over [0, M), each at a varying
    offset inside its stretch, always with the first and the last row."""
    step = max(1, M // max(count - 2, 1))
    rows = {0, M - 1}
    for i, lo in enumerate(range(0, M, step)):
        n = min(M, lo + step) - lo
        rows.add(lo + (i * 131 + 7 + salt) % n)
    return np.array(sorted(rows), np.int64)
