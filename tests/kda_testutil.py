"""Small helpers shared by the tests (input plumbing and error metrics only)."""
from __future__ import annotations

import numpy as np
import torch


def bf16_bits_exact(x) -> np.ndarray:
    """uint16 bf16 bit patterns of values that bf16 represents exactly."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    if not np.array_equal(back, a, equal_nan=True):
        raise ValueError("value not exactly representable in bf16")
    return bits


def bf16_tensor(x) -> torch.Tensor:
    """A torch bfloat16 CPU tensor holding values bf16 represents exactly."""
    bits = bf16_bits_exact(x)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)


def errors(got, ref):
    """(relative L2 error, max abs error) of ``got`` against ``ref``."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    nref = float(np.sqrt(np.sum(ref * ref)))
    rel = float(np.sqrt(np.sum(diff * diff))) / nref if nref > 0 else 0.0
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    return rel, mx


def rand_inputs(B, T, H, K, V, seed, *, init=None, varlen=None, gate_params=True):
    """Random small inputs (unit-norm q, k) as CPU torch tensors."""
    gen = torch.Generator().manual_seed(seed)
    cu = None
    if varlen is not None:
        lens = torch.tensor(varlen, dtype=torch.int64)
        cu = torch.zeros(len(varlen) + 1, dtype=torch.int64)
        cu[1:] = torch.cumsum(lens, 0)
        B, T = 1, int(cu[-1])

    def unit(shape):
        x = torch.randn(*shape, generator=gen)
        return (x / x.norm(dim=-1, keepdim=True)).bfloat16()

    q = unit((B, T, H, K))
    k = unit((B, T, H, K))
    v = torch.randn(B, T, H, V, generator=gen).bfloat16()
    g = torch.randn(B, T, H, K, generator=gen).bfloat16()
    beta = torch.randn(B, T, H, generator=gen).bfloat16()
    A_log = dt = None
    if gate_params:
        A_log = torch.log(torch.rand(H, generator=gen) * 15 + 1)
        dt = torch.randn(H, K, generator=gen)
    S0 = None
    if init is not None:
        N = B if cu is None else len(varlen)
        S0 = (0.1 * torch.randn(N, H, V, K, generator=gen)).to(init)
    return dict(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt,
                initial_state=S0, cu_seqlens=cu)
