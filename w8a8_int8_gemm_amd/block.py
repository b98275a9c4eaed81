"""One DiT block's six W8A8 projections, composed from library calls.

Data flow of a block (the six quantized Linears of "feat(mps): support
MiniMax-H3 INT8 inference on Apple M5", LightX2V pull request #1672,
description): Q, K and V share one per-token quantization of the block
input; the attention output projection and FC1 each quantize their own
input; FC2 takes SiLU of FC1's BF16 output, quantized ("MLX implementation
and experiment report", "What the default preserves": SiLU applied to the
BF16 value, rounded per the original recipe).  Attention and the norms are
not part of the projection path, so the synthetic block feeds its input X
to O and FC1 as well; that keeps four quantizations per block, as in the
model.  Everything here is a sequence of library calls on one stream;
outputs and scratch are preallocated once per token count.  The pages' own
H3 shapes (see datagen) use SwiGLU over a fused gate | up FC1 and feed V's
output (the attention result's shape) to the attention output projection.

Fused QKV (optional): the Q, K and V weights concatenated along the output
channels, [3N, K] with their scales and biases, run as one GEMM on the
shared quantized input.  Every output column depends only on its own weight
row, so the three column blocks of the fused output equal the separate
outputs bit for bit; the larger N fills the chip in fewer, fuller waves.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import binding as B
from . import datagen as D


def to_device_bf16(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to(device)


def from_device_bf16(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class DeviceProj:
    name: str
    N: int
    K: int
    w: object      # int8 [N, K]
    sw: object     # float32 [N]
    bias: object   # bf16 [N]


def upload_proj(p: D.Proj, pp: D.ProjParams, device="cuda") -> DeviceProj:
    import torch
    return DeviceProj(p.name, p.N, p.K,
                      torch.from_numpy(pp.w).to(device),
                      torch.from_numpy(pp.sw).to(device),
                      to_device_bf16(pp.bias, device))


def fuse_qkv(projs: dict) -> dict:
    """Replace projs' q, k, v by one "qkv" projection [3N, K] (device
    tensors concatenated along the output channels)."""
    import torch
    q, k, v = projs["q"], projs["k"], projs["v"]
    assert q.K == k.K == v.K
    fused = DeviceProj("qkv", q.N + k.N + v.N, q.K,
                       torch.cat([q.w, k.w, v.w]), torch.cat([q.sw, k.sw, v.sw]),
                       torch.cat([q.bias, k.bias, v.bias]))
    out = {n: p for n, p in projs.items() if n not in ("q", "k", "v")}
    out["qkv"] = fused
    return out


class BlockRunner:
    """Preallocated buffers for one token count M and one block layout
    (``projs``: the workload's six projections; ``mlp``: "silu", or
    "swiglu" for a fused gate | up FC1; ``o_input``: "x", or "v" to feed
    V's output to the attention output projection).  ``run`` enqueues the
    block's kernels on the current stream (or ``stream``).  ``on_gemm`` is
    called around every GEMM launch and ``on_quant`` around every
    quantization (for per-kernel event timing), as ``f(name, phase)``."""

    def __init__(self, M: int, device="cuda", fused_qkv: bool = False,
                 projs=D.BLOCK_PROJS, mlp: str = "silu", o_input: str = "x"):
        import torch
        if fused_qkv and o_input != "x":
            raise ValueError("fused QKV needs the block input as O's input")
        self.M, self.mlp, self.o_input = M, mlp, o_input
        shape = {p.name: (p.N, p.K) for p in projs}
        H = shape["q"][1]  # block width
        e = lambda *s, dt: torch.empty(s, dtype=dt, device=device)
        # X quantized for Q/K/V, for O (when it reads X) and for FC1
        self.xq = [e(M, H, dt=torch.int8) for _ in range(3)]
        self.xs = [e(M, dt=torch.float32) for _ in range(3)]
        self.oq = (e(M, shape["o"][1], dt=torch.int8) if o_input == "v"
                   else None)
        self.hq = e(M, shape["fc2"][1], dt=torch.int8)
        self.hs = e(M, dt=torch.float32)
        self.out = {n: e(M, shape[n][0], dt=torch.bfloat16)
                    for n in ("o", "fc1", "fc2")}
        if fused_qkv:
            nq = shape["q"][0]
            self.out["qkv"] = e(M, 3 * nq, dt=torch.bfloat16)
            for i, n in enumerate(("q", "k", "v")):
                self.out[n] = self.out["qkv"][:, i * nq:(i + 1) * nq]
        else:
            for n in ("q", "k", "v"):
                self.out[n] = e(M, shape[n][0], dt=torch.bfloat16)
        need = [B.gemm_workspace_bytes(M, N, K) for N, K in shape.values()]
        need.append(B.gemm_workspace_bytes(M, 3 * shape["q"][0], H))
        self.ws = e(max(max(need), 256), dt=torch.uint8)

    def _gemm(self, projs, name, q, s, stream, on_gemm):
        p = projs[name]
        if on_gemm:
            on_gemm(name, "begin")
        B.gemm(q, s, p.w, p.sw, p.bias, out=self.out[name],
               workspace=self.ws, stream=stream)
        if on_gemm:
            on_gemm(name, "end")

    def run_gemms(self, projs: dict, stream=None, on_gemm=None):
        """Only the block's GEMM calls, on the codes and scales the last
        ``run`` left in the buffers (GEMM timing)."""
        for n in (("qkv",) if "qkv" in projs else ("q", "k", "v")):
            self._gemm(projs, n, self.xq[0], self.xs[0], stream, on_gemm)
        self._gemm(projs, "o", self.oq if self.o_input == "v" else self.xq[1],
                   self.xs[1], stream, on_gemm)
        self._gemm(projs, "fc1", self.xq[2], self.xs[2], stream, on_gemm)
        self._gemm(projs, "fc2", self.hq, self.hs, stream, on_gemm)
        return self.out

    def codes_by_projection(self, projs: dict) -> dict:
        """The INT8 input codes each projection of ``projs`` read in the
        last ``run`` (the buffers, not copies)."""
        src = {"q": self.xq[0], "k": self.xq[0], "v": self.xq[0],
               "qkv": self.xq[0],
               "o": self.oq if self.o_input == "v" else self.xq[1],
               "fc1": self.xq[2], "fc2": self.hq}
        return {n: src[n] for n in projs}

    def run(self, x, projs: dict, stream=None, on_gemm=None,
            x_quantized: bool = False, on_quant=None):
        """x: bf16 [M, H].  Returns the dict of BF16 outputs.  With
        ``x_quantized`` the buffers ``xq[0]``, ``xs[0]`` already hold the
        quantization of x (written together with x by
        ``pow2_renorm_quantize`` between blocks) and Q, K and V use them."""
        def gemm(name, q, s):
            self._gemm(projs, name, q, s, stream, on_gemm)

        def quant(name, fn, *a, **kw):
            if on_quant:
                on_quant(name, "begin")
            fn(*a, stream=stream, **kw)
            if on_quant:
                on_quant(name, "end")

        # Q, K, V: one shared quantization of the block input (and, fused,
        # one GEMM over the concatenated weights).
        if not x_quantized:
            quant("quant", B.quantize_act, x, out=(self.xq[0], self.xs[0]))
        for n in (("qkv",) if "qkv" in projs else ("q", "k", "v")):
            gemm(n, self.xq[0], self.xs[0])
        # attention output projection and FC1 quantize their own inputs.
        if self.o_input == "v":
            quant("quant_o", B.quantize_act, self.out["v"],
                  out=(self.oq, self.xs[1]))
            gemm("o", self.oq, self.xs[1])
        else:
            quant("quant", B.quantize_act, x, out=(self.xq[1], self.xs[1]))
            gemm("o", self.xq[1], self.xs[1])
        quant("quant", B.quantize_act, x, out=(self.xq[2], self.xs[2]))
        gemm("fc1", self.xq[2], self.xs[2])
        # FC2 input: SiLU (or SwiGLU of gate | up) of FC1's BF16 output,
        # quantized in the same pass.
        if self.mlp == "swiglu":
            quant("swiglu_quant", B.quantize_act_swiglu, self.out["fc1"],
                  out=(self.hq, self.hs))
        else:
            quant("silu_quant", B.quantize_act, self.out["fc1"], silu=True,
                  out=(self.hq, self.hs))
        gemm("fc2", self.hq, self.hs)
        return self.out
