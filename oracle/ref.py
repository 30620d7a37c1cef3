"""Python entry points of the fp64 CPU oracle for the KDA forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The GPU library never imports
it, and nothing here calls the GPU library.

Two independent implementations of the same definition live here:

* :func:`kda_oracle` drives the plain C token loop in ``kda_ref.c`` (threads
  over (sequence, head) chains) and is what parity is measured against;
* :func:`kda_oracle_np` is a numpy token loop for tiny inputs, written apart
  from the C code so that each catches slips in the other.

The definition (see the header of ``kda_ref.c`` for the page citations):
per token, ``alpha = exp(lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h])))``,
``beta = sigmoid(beta_logit)``, decay ``S <- diag(alpha) S``, delta write
``S <- S + beta k (v - S^T k)^T``, read ``o = scale * S^T q``.  The state is
``S[k, v]``; the stored initial/final state is ``[.., V, K]``, i.e. ``S^T``.

Inputs are the exact values the GPU sees: bf16 tensors are given as torch
bfloat16 CPU tensors or as numpy uint16 arrays of bf16 bit patterns; A_log and
dt_bias are float32; cu_seqlens is int64.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence

import numpy as np

from . import build as _build

_STATE_NONE, _STATE_BF16, _STATE_FP32 = 0, 1, 2
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIBRARY):
        _build.build()
    lib = ctypes.CDLL(_build.LIBRARY)
    f = lib.kda_oracle_chains
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    f.argtypes = [p, p, p, p, p, ctypes.c_double, p, p, ctypes.c_double,
                  p, ctypes.c_int, p, i64, i64, i64, i64, p, p, i64, p, p,
                  ctypes.c_int]
    f.restype = ctypes.c_int
    _lib = lib
    return lib


# ----------------------------------------------------------------------------
# input plumbing (no arithmetic of the method)
# ----------------------------------------------------------------------------

def _bf16_bits(x) -> np.ndarray:
    """Return the bf16 bit patterns of ``x`` as a C-contiguous uint16 array."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("numpy bf16 inputs must be uint16 bit patterns")
        return np.ascontiguousarray(x)
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16:
        raise TypeError("expected a torch.bfloat16 tensor or a uint16 array")
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _f32(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.float32)
    import torch
    if x.dtype != torch.float32:
        raise TypeError("A_log / dt_bias must be float32")
    return x.detach().cpu().contiguous().numpy()


def _state(x):
    """Return (array, dtype tag) for an initial state given as bf16 or fp32."""
    if x is None:
        return None, _STATE_NONE
    if isinstance(x, np.ndarray):
        if x.dtype == np.uint16:
            return np.ascontiguousarray(x), _STATE_BF16
        if x.dtype == np.float32:
            return np.ascontiguousarray(x), _STATE_FP32
        raise TypeError("numpy initial_state must be uint16 (bf16 bits) or float32")
    import torch
    if x.dtype == torch.bfloat16:
        return _bf16_bits(x), _STATE_BF16
    if x.dtype == torch.float32:
        return x.detach().cpu().contiguous().numpy(), _STATE_FP32
    raise TypeError("initial_state must be bfloat16 or float32")


def _cu(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    if not isinstance(x, np.ndarray):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.int64)


def _segments(B: int, T: int, cu: Optional[np.ndarray]):
    """(number of sequences, [(t_begin, t_end, batch row)]) for the layout."""
    if cu is None:
        return B, [(0, T, b) for b in range(B)]
    return len(cu) - 1, [(int(cu[n]), int(cu[n + 1]), 0) for n in range(len(cu) - 1)]


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# the C oracle
# ----------------------------------------------------------------------------

def kda_oracle(q, k, v, g, beta, scale: float, A_log, dt_bias, lower_bound: float,
               initial_state=None, cu_seqlens=None,
               chains: Optional[Iterable[Sequence[int]]] = None,
               threads: Optional[int] = None, want_final: bool = True):
    """Run the fp64 token recurrence in C.

    With ``chains=None`` every (sequence, head) chain is computed and the
    result is ``(out, final)``: ``out`` fp64 ``[B,T,H,V]`` (varlen: ``[1,T,H,V]``,
    positions outside every segment left 0) and ``final`` fp64 ``[N,H,V,K]``
    (``None`` if ``want_final`` is false).

    With ``chains=[(n, h), ...]`` only those chains run and the result is a
    list of ``(out_chain [L_n, V], final_chain [V, K] or None)``.
    """
    qb, kb, vb, gb, bb = (_bf16_bits(x) for x in (q, k, v, g, beta))
    B, T, H, K = qb.shape
    V = vb.shape[-1]
    if kb.shape != (B, T, H, K) or gb.shape != (B, T, H, K):
        raise ValueError("q, k, g must share the shape [B,T,H,K]")
    if vb.shape != (B, T, H, V) or bb.shape != (B, T, H):
        raise ValueError("v must be [B,T,H,V] and beta [B,T,H]")
    a_log, dtb = _f32(A_log), _f32(dt_bias)
    if a_log is not None and a_log.shape != (H,):
        raise ValueError("A_log must be [H]")
    if dtb is not None and dtb.shape != (H, K):
        raise ValueError("dt_bias must be [H,K]")
    init, init_tag = _state(initial_state)
    cu = _cu(cu_seqlens)
    if cu is not None and B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    N, segs = _segments(B, T, cu)
    if init is not None and init.shape != (N, H, V, K):
        raise ValueError("initial_state must be [N,H,V,K]")

    full = chains is None
    if full:
        chain_list = [(n, h) for n in range(N) for h in range(H)]
    else:
        chain_list = [(int(n), int(h)) for n, h in chains]
        for n, h in chain_list:
            if not (0 <= n < N and 0 <= h < H):
                raise ValueError(f"chain {(n, h)} out of range")
    lengths = [segs[n][1] - segs[n][0] for n, _ in chain_list]
    offsets = np.zeros(len(chain_list), dtype=np.int64)
    if chain_list:
        offsets[1:] = np.cumsum(lengths)[:-1]
    chain_arr = np.ascontiguousarray(np.array(chain_list, dtype=np.int64).reshape(-1, 2))
    out_rows = np.zeros((int(sum(lengths)), V), dtype=np.float64)
    final = np.zeros((len(chain_list), V, K), dtype=np.float64) if want_final else None

    if threads is None:
        threads = len(os.sched_getaffinity(0))
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = _load().kda_oracle_chains(
        ptr(qb), ptr(kb), ptr(vb), ptr(gb), ptr(bb), float(scale), ptr(a_log), ptr(dtb),
        float(lower_bound), ptr(init), init_tag, ptr(cu), T, H, K, V,
        ptr(chain_arr), ptr(offsets), len(chain_list), ptr(out_rows), ptr(final),
        int(threads))
    if rc != 0:
        raise RuntimeError("oracle could not run every chain")

    if not full:
        res = []
        for i, L in enumerate(lengths):
            o = out_rows[offsets[i]:offsets[i] + L]
            res.append((o, None if final is None else final[i]))
        return res

    out = np.zeros((B, T, H, V), dtype=np.float64)
    for i, (n, h) in enumerate(chain_list):
        t0, t1, b = segs[n]
        out[b, t0:t1, h, :] = out_rows[offsets[i]:offsets[i] + lengths[i]]
    fin = None if final is None else final.reshape(N, H, V, K)
    return out, fin


# ----------------------------------------------------------------------------
# the numpy twin (tiny inputs only)
# ----------------------------------------------------------------------------

def _logistic_np(x: np.ndarray) -> np.ndarray:
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def kda_oracle_np(q, k, v, g, beta, scale: float, A_log, dt_bias, lower_bound: float,
                  initial_state=None, cu_seqlens=None):
    """Same definition as :func:`kda_oracle`, as a numpy loop over tokens.

    Returns ``(out [B,T,H,V], final [N,H,V,K])`` in fp64.
    """
    qf, kf, vf, gf, bf = (_bf16_to_f64(_bf16_bits(x)) for x in (q, k, v, g, beta))
    B, T, H, K = qf.shape
    V = vf.shape[-1]
    a_log, dtb = _f32(A_log), _f32(dt_bias)
    head_mult = np.ones(H) if a_log is None else np.exp(a_log.astype(np.float64))
    bias = np.zeros((H, K)) if dtb is None else dtb.astype(np.float64)
    init, tag = _state(initial_state)
    if tag == _STATE_BF16:
        init = _bf16_to_f64(init)
    elif tag == _STATE_FP32:
        init = init.astype(np.float64)
    cu = _cu(cu_seqlens)
    N, segs = _segments(B, T, cu)

    out = np.zeros((B, T, H, V))
    final = np.zeros((N, H, V, K))
    for n, (t0, t1, b) in enumerate(segs):
        for h in range(H):
            S = np.zeros((K, V)) if init is None else init[n, h].T.copy()
            for t in range(t0, t1):
                x = head_mult[h] * (gf[b, t, h] + bias[h])
                alpha = np.exp(lower_bound * _logistic_np(x))
                be = _logistic_np(np.array([bf[b, t, h]]))[0]
                kt, vt, qt = kf[b, t, h], vf[b, t, h], qf[b, t, h]
                S = alpha[:, None] * S
                S = S + be * np.outer(kt, vt - S.T @ kt)
                out[b, t, h] = scale * (S.T @ qt)
            final[n, h] = S.T
    return out, final
