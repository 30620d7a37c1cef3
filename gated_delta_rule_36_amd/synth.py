"""Seeded synthetic inputs for the KDA forward pass.

This module only draws random inputs; it holds none of the method's
arithmetic, and both the GPU path's tests and the CPU oracle's tests take
their inputs from here.

Recipe (the same for every workload; the pages run no dataset or public
benchmark, so every input is synthetic):

* a ``torch.Generator`` on the drawing device (the CPU by default, the GPU
  for the large workloads, where CPU drawing takes minutes) seeded with
  ``seed`` (0 unless stated), drawn in the fixed order: [sequence lengths],
  q, k, v, g, beta logits, A_log, dt_bias, [initial_state].  The same seed
  gives the same values on the same kind of device;
* the four ``[B,T,H,128]`` tensors are drawn one batch row at a time, so a
  large workload never holds more than one fp32 row in host memory;
* q, k ~ N(0,1), divided by their L2 norm over the 128 channels of each
  (token, head) row, then rounded to bf16;
* v, g ~ N(0,1) rounded to bf16;  beta logits ~ N(0,1) ``[B,T,H]`` in bf16;
* A_log = log(U(1,16)) fp32 ``[H]``;  dt_bias ~ N(0,1) fp32 ``[H,128]``;
* initial_state ~ N(0, 0.1^2) (standard deviation 0.1) in the stated dtype,
  ``[N,H,V,K]``;
* varlen lengths ~ U{100..4000}; a length divisible by 16 is reduced by one,
  so no sequence is a whole number of 16-token chunks;
* scale = 1/sqrt(128).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

HEAD_DIM = 128


@dataclasses.dataclass
class KdaInputs:
    """One workload's inputs, on the device they were drawn on (move with :meth:`to`)."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    A_log: Optional[torch.Tensor]
    dt_bias: Optional[torch.Tensor]
    scale: float
    lower_bound: float
    initial_state: Optional[torch.Tensor] = None
    cu_seqlens: Optional[torch.Tensor] = None
    final_dtype: Optional[torch.dtype] = None

    @property
    def num_seqs(self) -> int:
        return self.q.shape[0] if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    @property
    def head_tokens(self) -> int:
        B, T, H, _ = self.q.shape
        return B * T * H

    def to(self, device) -> "KdaInputs":
        mv = lambda t: None if t is None else t.to(device)
        return dataclasses.replace(
            self, q=mv(self.q), k=mv(self.k), v=mv(self.v), g=mv(self.g),
            beta=mv(self.beta), A_log=mv(self.A_log), dt_bias=mv(self.dt_bias),
            initial_state=mv(self.initial_state), cu_seqlens=mv(self.cu_seqlens))


def _rows(gen, B, T, H, D, unit_rows: bool) -> torch.Tensor:
    out = torch.empty(B, T, H, D, dtype=torch.bfloat16, device=gen.device)
    for b in range(B):
        x = torch.randn(T, H, D, generator=gen, device=gen.device)
        if unit_rows:
            x = x / x.norm(dim=-1, keepdim=True)
        out[b] = x.to(torch.bfloat16)
    return out


def make_inputs(B: int, T: int, H: int, *, lower_bound: float, seed: int = 0,
                K: int = HEAD_DIM, V: int = HEAD_DIM,
                seq_lengths: Optional[list] = None,
                varlen: Optional[tuple] = None,
                init_dtype: Optional[torch.dtype] = None,
                final_dtype: Optional[torch.dtype] = None,
                with_gate_params: bool = True,
                scale: Optional[float] = None,
                device: str = "cpu") -> KdaInputs:
    """Draw one workload.

    ``varlen=(N, lo, hi)`` draws N lengths in U{lo..hi} (first in the draw
    order) and packs them into one row (B must be 1, T is ignored);
    ``seq_lengths`` packs the given lengths instead.  ``init_dtype`` adds an
    initial state of that dtype; ``final_dtype`` records the dtype the caller
    wants ``final_state`` in.  Tensors are drawn on, and returned on,
    ``device``; sequence lengths are always drawn on the CPU.
    """
    gen = torch.Generator(device=device).manual_seed(seed)
    cpu_gen = gen if gen.device.type == "cpu" else torch.Generator().manual_seed(seed)
    cu = None
    if varlen is not None or seq_lengths is not None:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        if varlen is not None:
            n, lo, hi = varlen
            lens = torch.randint(lo, hi + 1, (n,), generator=cpu_gen)
            lens = torch.where(lens % 16 == 0, lens - 1, lens)
        else:
            lens = torch.tensor(seq_lengths, dtype=torch.int64)
        cu = torch.zeros(lens.numel() + 1, dtype=torch.int64)
        cu[1:] = torch.cumsum(lens, 0)
        T = int(cu[-1])
        cu = cu.to(device)
    q = _rows(gen, B, T, H, K, unit_rows=True)
    k = _rows(gen, B, T, H, K, unit_rows=True)
    v = _rows(gen, B, T, H, V, unit_rows=False)
    g = _rows(gen, B, T, H, K, unit_rows=False)
    dev = gen.device
    beta = torch.randn(B, T, H, generator=gen, device=dev).to(torch.bfloat16)
    A_log = dt_bias = None
    if with_gate_params:
        A_log = torch.log(torch.rand(H, generator=gen, device=dev) * 15.0 + 1.0)
        dt_bias = torch.randn(H, K, generator=gen, device=dev)
    init = None
    if init_dtype is not None:
        N = B if cu is None else cu.numel() - 1
        init = (0.1 * torch.randn(N, H, V, K, generator=gen, device=dev)).to(init_dtype)
    return KdaInputs(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt_bias,
                     scale=(1.0 / math.sqrt(K)) if scale is None else scale,
                     lower_bound=lower_bound, initial_state=init, cu_seqlens=cu,
                     final_dtype=final_dtype)


# The named workloads (seed 0 each).
WORKLOADS = {
    "tiny_b1_t64_h2": dict(B=1, T=64, H=2, lower_bound=-5.0),
    "small_b2_t128_h8": dict(B=2, T=128, H=8, lower_bound=-5.0),
    "long_b1_t8192_h16_state": dict(B=1, T=8192, H=16, lower_bound=-3.0,
                                    init_dtype=torch.float32, final_dtype=torch.float32),
    "varlen_n8_h32_bf16state": dict(B=1, T=0, H=32, lower_bound=-5.0, varlen=(8, 100, 4000),
                                    init_dtype=torch.bfloat16, final_dtype=torch.bfloat16),
    "large_b8_t16384_h32": dict(B=8, T=16384, H=32, lower_bound=-5.0,
                                final_dtype=torch.float32),
    # decode-shaped calls: a few new tokens per sequence, the fp32 state
    # carried in and out (the state traffic dominates)
    "decode_b64_t1_h32_state": dict(B=64, T=1, H=32, lower_bound=-5.0,
                                    init_dtype=torch.float32, final_dtype=torch.float32),
    "decode_b64_t8_h32_state": dict(B=64, T=8, H=32, lower_bound=-5.0,
                                    init_dtype=torch.float32, final_dtype=torch.float32),
    "decode_b64_t15_h32_state": dict(B=64, T=15, H=32, lower_bound=-5.0,
                                     init_dtype=torch.float32, final_dtype=torch.float32),
}


def workload(name: str, seed: int = 0, device: str = "cpu") -> KdaInputs:
    """Draw one of the named workloads on ``device``."""
    return make_inputs(**WORKLOADS[name], seed=seed, device=device)
