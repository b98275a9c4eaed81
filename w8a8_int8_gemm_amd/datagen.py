"""Seeded synthetic inputs for the W8A8 projection workloads.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the HIP path (benchmark, GPU tests) and the CPU oracle
(tests, CPU baseline) take their inputs from here, as host numpy arrays:

* activations X: BF16 [M, K], standard normal in FP32, then each entry,
  independently with probability 0.001, multiplied by 20 (outliers), then
  converted to BF16 with round-to-nearest-even (torch's CPU cast);
* weights W: INT8 [N, K] uniform on [-127, 127];
* per-output-channel weight scales: FP32 [N], exp(N(-6, 0.3^2)) drawn in
  binary64 and cast to FP32 (finite and > 0 by construction, asserted);
* bias: BF16 [N], N(0, 0.02^2) (0.02 is the standard deviation).

Every array has its own numpy PCG64 stream keyed by
``(seed, block, projection index, kind)`` so any single tensor can be
regenerated without drawing the others.  The shapes are those of one
block of a MiniMax-H3-style DiT at hidden width 5376: Q, K, V and the
attention output map 5376 -> 5376, FC1 maps 5376 -> 21504 and FC2 maps
21504 -> 5376 ("feat(mps): support MiniMax-H3 INT8 inference on Apple
M5", description: the six quantized Linears per block over 50 blocks).
Token counts follow the canvas rules of the h3.c article ("Resoluções e
durações": sides multiple of 32, at most 768*1344 pixels) and the latent
frame counts of the FastVideo pull request ("Test Results": 124 frames
give 37 video latent frames and 207 audio latent frames): one video latent
frame holds (H/32)*(W/32) tokens, so 544x960 gives 37*510 + 207 = 19077
tokens and 768x1344 gives 37*1008 + 207 = 37503.

A second shape set follows the pages' own H3 operator shapes ("MLX
implementation and experiment report", "Operator tuning": QKV 5376 ->
21504, i.e. 3 x 7168 = 56 heads x 128, a fused gate/up projection 5376 ->
28672 and a down projection 14336 -> 5376): Q, K, V map 5376 -> 7168, the
attention output 7168 -> 5376, FC1 (gate | up) 5376 -> 28672 and FC2
14336 -> 5376 after SwiGLU.  Attention is not on the projection path, so
that block feeds V's output to the attention output projection as the
stand-in for the attention result (same shape).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

HIDDEN = 5376
FFN = 21504
ATTN = 7168       # 56 heads x 128 (page shapes)
GATE_UP = 28672   # fused gate | up (page shapes)

KIND_X, KIND_W, KIND_SW, KIND_BIAS = 0, 1, 2, 3


@dataclass(frozen=True)
class Proj:
    name: str
    index: int
    N: int
    K: int


BLOCK_PROJS = (
    Proj("q", 0, HIDDEN, HIDDEN),
    Proj("k", 1, HIDDEN, HIDDEN),
    Proj("v", 2, HIDDEN, HIDDEN),
    Proj("o", 3, HIDDEN, HIDDEN),
    Proj("fc1", 4, FFN, HIDDEN),
    Proj("fc2", 5, HIDDEN, FFN),
)


PAGE_BLOCK_PROJS = (
    Proj("q", 0, ATTN, HIDDEN),
    Proj("k", 1, ATTN, HIDDEN),
    Proj("v", 2, ATTN, HIDDEN),
    Proj("o", 3, HIDDEN, ATTN),
    Proj("fc1", 4, GATE_UP, HIDDEN),
    Proj("fc2", 5, HIDDEN, GATE_UP // 2),
)


def tokens(height: int, width: int, video_latent_frames: int = 37,
           audio_tokens: int = 207) -> int:
    """Packed audio/video token count of one DiT input."""
    assert height % 32 == 0 and width % 32 == 0
    return video_latent_frames * (height // 32) * (width // 32) + audio_tokens


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    projs: tuple
    blocks: int
    seed: int
    mlp: str = "silu"     # FC1 -> FC2 glue: "silu" or "swiglu" (gate | up)
    o_input: str = "x"    # attention output projection input: "x" or "v"


WORKLOADS = {
    0: Workload("single_q_projection_m64", 64, (BLOCK_PROJS[0],), 1, 0),
    1: Workload("dit_block_m4096", 4096, BLOCK_PROJS, 1, 1),
    2: Workload("dit_block_544x960_124f", tokens(544, 960), BLOCK_PROJS, 1, 2),
    3: Workload("dit_block_768x1344_124f", tokens(768, 1344), BLOCK_PROJS, 1, 3),
    4: Workload("dit_sweep_300_linears_544x960_124f", tokens(544, 960),
                BLOCK_PROJS, 50, 4),
    5: Workload("dit_block_h3_page_shapes_544x960_124f", tokens(544, 960),
                PAGE_BLOCK_PROJS, 1, 5, "swiglu", "v"),
    6: Workload("dit_sweep_300_linears_h3_page_shapes_544x960_124f",
                tokens(544, 960), PAGE_BLOCK_PROJS, 50, 6, "swiglu", "v"),
}


def rng(seed: int, block: int, proj: int, kind: int) -> np.random.Generator:
    return np.random.default_rng([seed, block, proj, kind])


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """FP32 -> BF16 bit patterns (uint16), round-to-nearest-even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def activations(M: int, K: int, seed: int, block: int = 0,
                proj: int = 0) -> np.ndarray:
    g = rng(seed, block, proj, KIND_X)
    x = g.standard_normal((M, K), dtype=np.float32)
    outlier = g.random((M, K), dtype=np.float32) < np.float32(0.001)
    x[outlier] *= np.float32(20.0)
    return to_bf16_bits(x)


def weights(N: int, K: int, seed: int, block: int = 0,
            proj: int = 0) -> np.ndarray:
    g = rng(seed, block, proj, KIND_W)
    return g.integers(-127, 127, size=(N, K), endpoint=True, dtype=np.int8)


def weight_scales(N: int, seed: int, block: int = 0,
                  proj: int = 0) -> np.ndarray:
    g = rng(seed, block, proj, KIND_SW)
    sw = np.exp(g.normal(-6.0, 0.3, N)).astype(np.float32)
    assert np.all(np.isfinite(sw)) and np.all(sw > 0)
    return sw


def bias(N: int, seed: int, block: int = 0, proj: int = 0) -> np.ndarray:
    g = rng(seed, block, proj, KIND_BIAS)
    return to_bf16_bits(g.normal(0.0, 0.02, N).astype(np.float32))


@dataclass
class ProjParams:
    w: np.ndarray      # int8 [N, K]
    sw: np.ndarray     # float32 [N]
    bias: np.ndarray   # uint16 [N]


def proj_params(p: Proj, seed: int, block: int = 0) -> ProjParams:
    return ProjParams(weights(p.N, p.K, seed, block, p.index),
                      weight_scales(p.N, seed, block, p.index),
                      bias(p.N, seed, block, p.index))


def block_params(wl: Workload, block: int = 0, threads: int = 8):
    """All projection parameters of one block, drawn in parallel threads."""
    with ThreadPoolExecutor(max(1, threads)) as ex:
        out = list(ex.map(lambda p: proj_params(p, wl.seed, block), wl.projs))
    return {p.name: pp for p, pp in zip(wl.projs, out)}


def row_sample(M: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct row indices for sampled checks; always includes the
    first and the last row (the ragged tail)."""
    count = min(count, M)
    g = np.random.default_rng([seed, 0x5A3])
    idx = set(g.choice(M, size=count, replace=False).tolist())
    idx.update({0, M - 1})
    return np.array(sorted(idx), np.int64)
